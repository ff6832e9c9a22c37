// gdr_api.cpp -- the C ABI declared in include/gdr.h: descriptor validation,
// workspace layout, and dispatch to the kernel launcher of the requested
// (io dtype, chunk, head dim, gate form).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <initializer_list>
#include <string>

#include "gdr.h"
#include "gdr_launch.hpp"

namespace {

thread_local std::string g_hip_msg;

size_t elem_bytes(int io) { return io == GDR_DTYPE_F32 ? 4 : 2; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t max_chunks(const gdr_bwd_desc_t* d) {
    const int64_t C = d->chunk;
    if (d->n_seqs > 0) return d->T / C + d->n_seqs;  // each sequence adds at most one partial chunk
    return d->B * ((d->T + C - 1) / C);
}

// Workspace regions in a fixed order (gdr_bwd_workspace_offsets reports them).
enum {
    WS_CTAB, WS_SEQOFF, WS_SAQKT, WS_AM, WS_AT, WS_W, WS_WT, WS_KT, WS_KTT, WS_UT, WS_QST,
    WS_GLAST, WS_H, WS_X, WS_DH, WS_T, WS_COUNT
};

void layout(const gdr_bwd_desc_t* d, size_t off[WS_COUNT + 1]) {
    const size_t nc = (size_t)max_chunks(d), H = d->H, C = d->chunk, D = d->K, es = elem_bytes(d->io_dtype);
    const size_t N = d->n_seqs > 0 ? d->n_seqs : d->B;
    size_t sz[WS_COUNT];
    sz[WS_CTAB] = nc * sizeof(gdr::ChunkEntry);
    sz[WS_SEQOFF] = (2 * N + 1) * sizeof(int);   // chunk offsets, then the longest-first order
    sz[WS_SAQKT] = sz[WS_AM] = nc * H * C * C * es;
    sz[WS_AT] = 0;   // kept in the order, empty: A^T is read from the staged A
    sz[WS_W] = sz[WS_WT] = sz[WS_KT] = sz[WS_KTT] = sz[WS_UT] = sz[WS_QST] = nc * H * C * D * es;
    sz[WS_GLAST] = nc * H * D * 4;
    sz[WS_H] = sz[WS_DH] = nc * H * D * D * es;
    sz[WS_X] = sz[WS_T] = nc * H * C * D * es;
    size_t o = 0;
    for (int i = 0; i < WS_COUNT; ++i) {
        off[i] = o;
        o += align256(sz[i]);
    }
    off[WS_COUNT] = o;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Required token buffers: non-null and 16-byte aligned, except that with no
// tokens at all (T == 0) they may be null (no kernel touches them then).
bool token_buffers_ok(const gdr_bwd_desc_t* d, std::initializer_list<const void*> ptrs) {
    for (const void* ptr : ptrs)
        if ((!ptr && d->T > 0) || !aligned16(ptr)) return false;
    return true;
}

}  // namespace

namespace gdr {
// Keeps the HIP error text of a failed call for gdr_strerror(GDR_EHIP).
void set_hip_error(const char* what, hipError_t e) {
    g_hip_msg = std::string("HIP error in ") + what + ": " + hipGetErrorString(e);
}
}  // namespace gdr

extern "C" {

int gdr_bwd_check(const gdr_bwd_desc_t* d) {
    if (!d) return GDR_EINVAL;
    if (d->B < 1 || d->T < 0 || d->H < 1 || d->Hg < 1 || d->K < 1 || d->V < 1) return GDR_EINVAL;
    if (d->H % d->Hg != 0) return GDR_EINVAL;
    if (d->gate != GDR_GATE_PER_CHANNEL && d->gate != GDR_GATE_SCALAR) return GDR_EINVAL;
    if (d->io_dtype < GDR_DTYPE_F32 || d->io_dtype > GDR_DTYPE_F16) return GDR_EINVAL;
    if (d->n_seqs < 0 || (d->n_seqs > 0 && d->B != 1)) return GDR_EINVAL;
    if (d->chunk < 1 || d->sub_chunk < 1) return GDR_EINVAL;
    if (d->state_v_first != 0 && d->state_v_first != 1) return GDR_EINVAL;
    // flattened token indices are 32-bit on the device
    if (d->B * d->T > (int64_t)INT32_MAX / 2) return GDR_EUNSUPPORTED;
    if (d->K != d->V || (d->K != 64 && d->K != 128)) return GDR_EUNSUPPORTED;
    if (d->chunk != 32 && d->chunk != 64) return GDR_EUNSUPPORTED;
    if (d->io_dtype == GDR_DTYPE_F32 && d->K != 64) return GDR_EUNSUPPORTED;
    if (d->sub_chunk != 16) return GDR_EUNSUPPORTED;
    if (max_chunks(d) * d->H > (int64_t)INT32_MAX / 2) return GDR_EUNSUPPORTED;
    return GDR_OK;
}

size_t gdr_bwd_workspace_bytes(const gdr_bwd_desc_t* d) {
    if (gdr_bwd_check(d) != GDR_OK) return 0;
    size_t off[WS_COUNT + 1];
    layout(d, off);
    return off[WS_COUNT];
}

// The fused reverse backward's workspace: the standard regions, then (GQA
// only) fp32 dq and dk partials per value head, [B*T][H][K] each.
static size_t fused_partial_bytes(const gdr_bwd_desc_t* d) {
    return d->H > d->Hg ? align256((size_t)(d->B * d->T) * d->H * d->K * 4) : 0;
}

size_t gdr_bwd_fused_workspace_bytes(const gdr_bwd_desc_t* d) {
    if (gdr_bwd_check(d) != GDR_OK || d->chunk != 32) return 0;
    size_t off[WS_COUNT + 1];
    layout(d, off);
    return off[WS_COUNT] + 2 * fused_partial_bytes(d);
}

int gdr_bwd_workspace_offsets(const gdr_bwd_desc_t* d, size_t* offsets, int n) {
    const int rc = gdr_bwd_check(d);
    if (rc != GDR_OK) return rc;
    if (!offsets || n < WS_COUNT + 1) return GDR_EINVAL;
    size_t off[WS_COUNT + 1];
    layout(d, off);
    for (int i = 0; i <= WS_COUNT; ++i) offsets[i] = off[i];
    return GDR_OK;
}

}  // extern "C"

// Checks shared by both passes and the parameter block (problem, workspace).
static int fill_params(const gdr_bwd_desc_t* d, const int32_t* cu_seqlens, void* workspace,
                       size_t workspace_bytes, gdr::Params& p) {
    int rc = gdr_bwd_check(d);
    if (rc != GDR_OK) return rc;
    if ((d->n_seqs > 0) != (cu_seqlens != nullptr)) return GDR_EINVAL;
    size_t off[WS_COUNT + 1];
    layout(d, off);
    if (!workspace || workspace_bytes < off[WS_COUNT]) return GDR_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return GDR_EINVAL;
    char* ws = static_cast<char*>(workspace);
    p = gdr::Params{};
    p.B = d->B;
    p.T = d->T;
    p.H = d->H;
    p.Hg = d->Hg;
    p.G = d->H / d->Hg;
    p.N = d->n_seqs > 0 ? d->n_seqs : (int)d->B;
    p.nc_max = (int)max_chunks(d);
    p.varlen = d->n_seqs > 0;
    p.vfirst = d->state_v_first;
    p.scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->K);
    p.cu = cu_seqlens;
    p.ctab = reinterpret_cast<gdr::ChunkEntry*>(ws + off[WS_CTAB]);
    p.seq_off = reinterpret_cast<int*>(ws + off[WS_SEQOFF]);
    p.seq_ord = p.seq_off + p.N + 1;
    p.sAqkT = ws + off[WS_SAQKT];
    p.Am = ws + off[WS_AM];
    p.w = ws + off[WS_W];
    p.wT = ws + off[WS_WT];
    p.kt = ws + off[WS_KT];
    p.ktT = ws + off[WS_KTT];
    p.uT = ws + off[WS_UT];
    p.qsT = ws + off[WS_QST];
    p.glast = reinterpret_cast<float*>(ws + off[WS_GLAST]);
    p.hbuf = ws + off[WS_H];
    p.xbuf = ws + off[WS_X];
    p.dhbuf = ws + off[WS_DH];
    p.tbuf = ws + off[WS_T];
    return GDR_OK;
}

static int launch(gdr::LaunchFn fn, const gdr::Params& p, void* stream, void* const* events) {
    if (!fn) return GDR_EUNSUPPORTED;
    hipError_t e = fn(p, static_cast<hipStream_t>(stream), reinterpret_cast<hipEvent_t const*>(events));
    if (e != hipSuccess) {
        g_hip_msg = std::string("HIP error: ") + hipGetErrorString(e);
        return GDR_EHIP;
    }
    return GDR_OK;
}

extern "C" {

int gdr_bwd_with_events(const gdr_bwd_desc_t* d, const void* q, const void* k, const void* v,
                        const float* g, const void* beta, const float* h0, const void* do_,
                        const float* dht, const int32_t* cu_seqlens, void* dq, void* dk, void* dv,
                        float* dg, void* db, float* dh0, void* workspace, size_t workspace_bytes,
                        void* stream, void* const* stage_events) {
    int rc = gdr_bwd_check(d);
    if (rc != GDR_OK) return rc;
    if (!token_buffers_ok(d, {q, k, v, g, beta, do_, dq, dk, dv, dg, db})) return GDR_EINVAL;
    if (!dh0 || !aligned16(dh0)) return GDR_EINVAL;
    if ((h0 && !aligned16(h0)) || (dht && !aligned16(dht))) return GDR_EINVAL;
    gdr::Params p;
    rc = fill_params(d, cu_seqlens, workspace, workspace_bytes, p);
    if (rc != GDR_OK) return rc;
    p.dirs = 2;
    p.dir0 = 0;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.dout = do_; p.dht = dht;
    p.dq = dq; p.dk = dk; p.dv = dv; p.dg = dg; p.db = db; p.dh0 = dh0;
    return launch(gdr::find_launcher(d->io_dtype, d->chunk, d->K, d->gate == GDR_GATE_SCALAR, 0), p,
                  stream, stage_events);
}

int gdr_fwd(const gdr_bwd_desc_t* d, const void* q, const void* k, const void* v, const float* g,
            const void* beta, const float* h0, const int32_t* cu_seqlens, void* o, float* ht,
            void* workspace, size_t workspace_bytes, void* stream) {
    int rc = gdr_bwd_check(d);
    if (rc != GDR_OK) return rc;
    if (!token_buffers_ok(d, {q, k, v, g, beta, o})) return GDR_EINVAL;
    if ((h0 && !aligned16(h0)) || (ht && !aligned16(ht))) return GDR_EINVAL;
    gdr::Params p;
    rc = fill_params(d, cu_seqlens, workspace, workspace_bytes, p);
    if (rc != GDR_OK) return rc;
    p.dirs = 1;
    p.dir0 = 0;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0;
    p.o = o; p.ht = ht;
    return launch(gdr::find_launcher(d->io_dtype, d->chunk, d->K, d->gate == GDR_GATE_SCALAR, 1), p,
                  stream, nullptr);
}

int gdr_bwd_after_fwd(const gdr_bwd_desc_t* d, const void* q, const void* k, const void* v,
                      const float* g, const void* beta, const void* do_, const float* dht,
                      const int32_t* cu_seqlens, void* dq, void* dk, void* dv, float* dg, void* db,
                      float* dh0, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = gdr_bwd_check(d);
    if (rc != GDR_OK) return rc;
    if (!token_buffers_ok(d, {q, k, v, g, beta, do_, dq, dk, dv, dg, db})) return GDR_EINVAL;
    if (!dh0 || !aligned16(dh0)) return GDR_EINVAL;
    if (dht && !aligned16(dht)) return GDR_EINVAL;
    gdr::Params p;
    rc = fill_params(d, cu_seqlens, workspace, workspace_bytes, p);
    if (rc != GDR_OK) return rc;
    p.dirs = 1;
    p.dir0 = 1;   // reverse sweep only: the forward's table, factors, h and X are in the workspace
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.dout = do_; p.dht = dht;
    p.dq = dq; p.dk = dk; p.dv = dv; p.dg = dg; p.db = db; p.dh0 = dh0;
    return launch(gdr::find_launcher(d->io_dtype, d->chunk, d->K, d->gate == GDR_GATE_SCALAR, 0), p,
                  stream, nullptr);
}

int gdr_bwd_from_states(const gdr_bwd_desc_t* d, const void* q, const void* k, const void* v,
                        const float* g, const void* beta, const void* do_, const float* dht,
                        const int32_t* cu_seqlens, const void* h, int64_t n_h_chunks, void* dq, void* dk,
                        void* dv, float* dg, void* db, float* dh0, void* workspace, size_t workspace_bytes,
                        void* stream) {
    int rc = gdr_bwd_check(d);
    if (rc != GDR_OK) return rc;
    if (!token_buffers_ok(d, {q, k, v, g, beta, do_, dq, dk, dv, dg, db, h})) return GDR_EINVAL;
    if (!dh0 || !aligned16(dh0)) return GDR_EINVAL;
    if (dht && !aligned16(dht)) return GDR_EINVAL;
    if (n_h_chunks < 0 || n_h_chunks > max_chunks(d)) return GDR_EINVAL;
    if (d->n_seqs == 0 && n_h_chunks != max_chunks(d)) return GDR_EINVAL;   // B ceil(T / C)
    gdr::Params p;
    rc = fill_params(d, cu_seqlens, workspace, workspace_bytes, p);
    if (rc != GDR_OK) return rc;
    p.dirs = 1;
    p.dir0 = 1;   // reverse sweep only: the states kernel stands in for the forward sweep
    p.hsrc = h;
    p.nh_src = (int)n_h_chunks;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.dout = do_; p.dht = dht;
    p.dq = dq; p.dk = dk; p.dv = dv; p.dg = dg; p.db = db; p.dh0 = dh0;
    return launch(gdr::find_launcher(d->io_dtype, d->chunk, d->K, d->gate == GDR_GATE_SCALAR, 0), p,
                  stream, nullptr);
}

int gdr_bwd_fused(const gdr_bwd_desc_t* d, const void* q, const void* k, const void* v, const float* g,
                  const void* beta, const float* h0, const void* do_, const float* dht,
                  const int32_t* cu_seqlens, void* dq, void* dk, void* dv, float* dg, void* db, float* dh0,
                  void* workspace, size_t workspace_bytes, void* stream) {
    int rc = gdr_bwd_check(d);
    if (rc != GDR_OK) return rc;
    if (d->chunk != 32) return GDR_EUNSUPPORTED;
    if (!token_buffers_ok(d, {q, k, v, g, beta, do_, dq, dk, dv, dg, db})) return GDR_EINVAL;
    if (!dh0 || !aligned16(dh0)) return GDR_EINVAL;
    if ((h0 && !aligned16(h0)) || (dht && !aligned16(dht))) return GDR_EINVAL;
    const size_t need = gdr_bwd_fused_workspace_bytes(d);
    if (!workspace || workspace_bytes < need) return GDR_EWORKSPACE;
    gdr::Params p;
    rc = fill_params(d, cu_seqlens, workspace, workspace_bytes, p);
    if (rc != GDR_OK) return rc;
    size_t off[WS_COUNT + 1];
    layout(d, off);
    char* ws = static_cast<char*>(workspace);
    p.dqp = reinterpret_cast<float*>(ws + off[WS_COUNT]);
    p.dkp = reinterpret_cast<float*>(ws + off[WS_COUNT] + fused_partial_bytes(d));
    p.dirs = 1;
    p.dir0 = 0;   // the forward sweep alone: the reverse one runs inside the fused kernel
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.dout = do_; p.dht = dht;
    p.dq = dq; p.dk = dk; p.dv = dv; p.dg = dg; p.db = db; p.dh0 = dh0;
    return launch(gdr::find_launcher(d->io_dtype, d->chunk, d->K, d->gate == GDR_GATE_SCALAR, 2), p,
                  stream, nullptr);
}

int gdr_bwd(const gdr_bwd_desc_t* d, const void* q, const void* k, const void* v, const float* g,
            const void* beta, const float* h0, const void* do_, const float* dht,
            const int32_t* cu_seqlens, void* dq, void* dk, void* dv, float* dg, void* db, float* dh0,
            void* workspace, size_t workspace_bytes, void* stream) {
    return gdr_bwd_with_events(d, q, k, v, g, beta, h0, do_, dht, cu_seqlens, dq, dk, dv, dg, db,
                               dh0, workspace, workspace_bytes, stream, nullptr);
}

const char* gdr_strerror(int status) {
    switch (status) {
        case GDR_OK: return "ok";
        case GDR_EINVAL: return "invalid argument (shape, null pointer or alignment)";
        case GDR_EUNSUPPORTED: return "unsupported configuration (K == V in {64,128}, K == 64 for fp32, chunk in {32,64}, sub_chunk 16)";
        case GDR_EWORKSPACE: return "workspace missing or smaller than gdr_bwd_workspace_bytes()";
        case GDR_EHIP: return g_hip_msg.empty() ? "HIP error" : g_hip_msg.c_str();
        case GDR_ESCRATCH:
            return "gdr_bwd_static: the problem needs more workspace than the library's fixed scratch "
                   "(GDR_STATIC_SCRATCH_BYTES); use gdr_bwd with a caller workspace";
        default: return "unknown status";
    }
}

const char* gdr_version(void) { return "0.2.0"; }

}  // extern "C"
