// maglev_api.cpp -- the exported C ABI (include/maglev.h): argument
// validation, status codes, the RoPE table cache and dispatch to the kernel
// launchers. No arithmetic of the method happens here apart from the host
// table of RoPE angles.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "internal.hpp"
#include "profile.hpp"

namespace maglev {
namespace {

thread_local std::string g_last_error;

maglev_status_t fail(maglev_status_t st, const char *msg)
{
    g_last_error = msg;
    return st;
}

maglev_status_t hip_status(hipError_t e)
{
    // debug mode: a failure seen after one of this call's launches names its kernel
    const char *kern = nullptr;
    hipError_t de = hipSuccess;
    if (prof::debug_take(&kern, &de)) {
        g_last_error = std::string(kern ? kern : "?") + ": " + hipGetErrorString(de);
        return MAGLEV_ERR_HIP;
    }
    if (e == hipSuccess) return MAGLEV_OK;
    g_last_error = hipGetErrorString(e);
    return MAGLEV_ERR_HIP;
}

// The status of a call that launched work on `s`; in debug mode also the
// check after its last launches (those outside a named kernel scope included).
maglev_status_t launched(hipStream_t s, hipError_t e)
{
    if (e == hipSuccess) prof::debug_after("end of call", s);
    return hip_status(e);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

maglev_status_t check_dtype(int dtype)
{
    if (dtype != MAGLEV_F32 && dtype != MAGLEV_BF16)
        return fail(MAGLEV_ERR_INVALID_VALUE, "dtype must be MAGLEV_F32 or MAGLEV_BF16");
    return MAGLEV_OK;
}

maglev_status_t check_geom(const maglev_geom_t *g, Geom *out)
{
    if (!g) return fail(MAGLEV_ERR_INVALID_VALUE, "geometry pointer is NULL");
    if (g->B < 0 || g->T < 0) return fail(MAGLEV_ERR_INVALID_VALUE, "B and T must be >= 0");
    if (g->H < 1) return fail(MAGLEV_ERR_INVALID_VALUE, "H must be >= 1");
    if (g->Dh != 64 && g->Dh != 128) return fail(MAGLEV_ERR_UNSUPPORTED, "Dh must be 64 or 128");
    // the attention passes address a tile of 32 token rows (H*Dh elements
    // apart) with 32-bit byte offsets
    if ((int64_t)g->H * g->Dh > 65536) return fail(MAGLEV_ERR_UNSUPPORTED, "H*Dh must be at most 65536");
    if (g->d < 16 || (g->d % 16) != 0)
        return fail(MAGLEV_ERR_INVALID_VALUE, "d must be a positive multiple of 16");
    if (g->W < 1) return fail(MAGLEV_ERR_INVALID_VALUE, "W must be >= 1");
    if (g->pos0 < 0) return fail(MAGLEV_ERR_INVALID_VALUE, "pos0 must be >= 0");
    if (!(g->scale == g->scale) || !(g->rope_base == g->rope_base))
        return fail(MAGLEV_ERR_INVALID_VALUE, "scale and rope_base must not be NaN");
    maglev_status_t st = check_dtype(g->dtype);
    if (st != MAGLEV_OK) return st;
    const double elems = (double)g->B * (double)g->T * (double)g->H * (double)g->Dh;
    const double melems = (double)g->B * (double)g->T * (double)g->d;
    if (elems > 4.0e12 || melems > 4.0e12 || (double)g->T > 2.0e9)
        return fail(MAGLEV_ERR_INVALID_VALUE, "tensor sizes out of range");
    out->B = g->B; out->T = g->T; out->H = g->H; out->Dh = g->Dh; out->d = g->d; out->W = g->W;
    out->pos0 = g->pos0;
    out->rope_base = g->rope_base;
    out->scale = g->scale > 0.0f ? g->scale : (float)(1.0 / sqrt((double)g->Dh));
    out->dtype = g->dtype;
    return MAGLEV_OK;
}

maglev_status_t check_ptrs(std::initializer_list<const void *> ptrs)
{
    for (const void *p : ptrs) {
        if (!p) return fail(MAGLEV_ERR_INVALID_VALUE, "a required pointer is NULL");
        if (!aligned16(p)) return fail(MAGLEV_ERR_MISALIGNED, "a pointer is not 16-byte aligned");
    }
    return MAGLEV_OK;
}

// ---- RoPE table cache --------------------------------------------------------
struct TableKey {
    int device, Dh;
    float base;
    bool operator<(const TableKey &o) const
    {
        return std::tie(device, Dh, base) < std::tie(o.device, o.Dh, o.base);
    }
};
struct TableEntry {
    float2 *ptr = nullptr;
    int64_t positions = 0;
};
std::mutex g_table_mu;
std::map<TableKey, TableEntry> g_tables;
std::vector<float2 *> g_retired;  // grown-out tables stay allocated: kernels may still read them

}  // namespace

maglev_status_t rope_table(int Dh, float base, int64_t max_pos, const float2 **table)
{
    *table = nullptr;
    if (!(base > 0.0f)) return MAGLEV_OK;
    if (max_pos < 1) max_pos = 1;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    std::lock_guard<std::mutex> lock(g_table_mu);
    TableEntry &ent = g_tables[TableKey{dev, Dh, base}];
    if (ent.positions >= max_pos) {
        *table = ent.ptr;
        return MAGLEV_OK;
    }
    int64_t n = ent.positions ? ent.positions : 4096;
    while (n < max_pos) n *= 2;
    const int half = Dh / 2;
    std::vector<float2> host((size_t)n * half);
    for (int i = 0; i < half; ++i) {
        const double theta = pow((double)base, -2.0 * (double)i / (double)Dh);
        for (int64_t p = 0; p < n; ++p) {
            const double phi = (double)p * theta;
            host[(size_t)p * half + i] = make_float2((float)cos(phi), (float)sin(phi));
        }
    }
    float2 *dptr = nullptr;
    e = hipMalloc(&dptr, host.size() * sizeof(float2));
    if (e != hipSuccess) return hip_status(e);
    e = hipMemcpy(dptr, host.data(), host.size() * sizeof(float2), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(dptr);
        return hip_status(e);
    }
    if (ent.ptr) g_retired.push_back(ent.ptr);
    ent.ptr = dptr;
    ent.positions = n;
    *table = dptr;
    return MAGLEV_OK;
}

namespace {

// Table lookup that refuses to allocate while the stream is being captured.
maglev_status_t table_for(const Geom &g, hipStream_t s, const float2 **table)
{
    *table = nullptr;
    if (!(g.rope_base > 0.0f)) return MAGLEV_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return hip_status(e);
    const int64_t need = g.pos0 + g.T;
    if (cs != hipStreamCaptureStatusNone) {
        std::lock_guard<std::mutex> lock(g_table_mu);
        int dev = 0;
        (void)hipGetDevice(&dev);
        auto it = g_tables.find(TableKey{dev, g.Dh, g.rope_base});
        if (it == g_tables.end() || it->second.positions < need)
            return fail(MAGLEV_ERR_UNSUPPORTED,
                        "RoPE table missing during stream capture: call maglev_prepare first");
        *table = it->second.ptr;
        return MAGLEV_OK;
    }
    return rope_table(g.Dh, g.rope_base, need, table);
}

}  // namespace
}  // namespace maglev

using namespace maglev;

extern "C" {

const char *maglev_status_string(maglev_status_t status)
{
    switch (status) {
    case MAGLEV_OK: return "MAGLEV_OK";
    case MAGLEV_ERR_INVALID_VALUE: return "MAGLEV_ERR_INVALID_VALUE";
    case MAGLEV_ERR_UNSUPPORTED: return "MAGLEV_ERR_UNSUPPORTED";
    case MAGLEV_ERR_MISALIGNED: return "MAGLEV_ERR_MISALIGNED";
    case MAGLEV_ERR_WORKSPACE: return "MAGLEV_ERR_WORKSPACE";
    case MAGLEV_ERR_HIP: return "MAGLEV_ERR_HIP";
    }
    return "MAGLEV_ERR_UNKNOWN";
}

const char *maglev_last_error(void) { return g_last_error.c_str(); }

int maglev_abi_version(void) { return MAGLEV_ABI_VERSION; }

maglev_status_t maglev_prepare(int32_t Dh, float rope_base, int64_t max_pos)
{
    if (Dh != 64 && Dh != 128) return fail(MAGLEV_ERR_UNSUPPORTED, "Dh must be 64 or 128");
    if (max_pos < 0) return fail(MAGLEV_ERR_INVALID_VALUE, "max_pos must be >= 0");
    // set-up of the current device: the address of the allocation-free
    // loss's scratch array, then the RoPE table
    float *scr = nullptr;
    maglev_status_t st = hip_status(loss_scratch_address(&scr));
    if (st != MAGLEV_OK) return st;
    const float2 *t = nullptr;
    return rope_table(Dh, rope_base, max_pos, &t);
}

maglev_status_t maglev_mem_project(const maglev_geom_t *g, int shift, const void *m,
                                   const void *W_Km, const void *W_Vm, const void *k,
                                   const void *v, const float *gate_logit, void *kmem,
                                   void *vmem, void *kmix, void *vmix, hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    if (shift != 0 && shift != 1) return fail(MAGLEV_ERR_INVALID_VALUE, "shift must be 0 or 1");
    if (G.N() == 0) return MAGLEV_OK;   // nothing to read or write (empty tensors may be null)
    const int nmix = (k != nullptr) + (v != nullptr) + (gate_logit != nullptr) +
                     (kmix != nullptr) + (vmix != nullptr);
    if (nmix != 0 && nmix != 5)
        return fail(MAGLEV_ERR_INVALID_VALUE, "k, v, gate_logit, kmix, vmix: give all or none");
    st = check_ptrs({m, W_Km, W_Vm, kmem, vmem});
    if (st != MAGLEV_OK) return st;
    const float2 *rope = nullptr;
    if (nmix) {
        st = check_ptrs({k, v, kmix, vmix});
        if (st != MAGLEV_OK) return st;
        st = table_for(G, stream, &rope);
        if (st != MAGLEV_OK) return st;
    }
    hipError_t e = launch_project(G, shift, m, W_Km, W_Vm, kmem, vmem, stream);
    if (e == hipSuccess && nmix)
        e = launch_mix(G, k, v, kmem, vmem, gate_logit, rope, kmix, vmix, stream);
    return launched(stream, e);
}

maglev_status_t maglev_swa_inject_fwd(const maglev_geom_t *g, const void *q, const void *kmix,
                                      const void *vmix, void *o, float *lse, hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    if (G.N() == 0) return MAGLEV_OK;   // nothing to read or write
    st = check_ptrs({q, kmix, vmix, o});
    if (st != MAGLEV_OK) return st;
    if (lse && !aligned16(lse)) return fail(MAGLEV_ERR_MISALIGNED, "lse is not 16-byte aligned");
    const float2 *rope = nullptr;
    st = table_for(G, stream, &rope);
    if (st != MAGLEV_OK) return st;
    return launched(stream, launch_attn_fwd(G, q, kmix, vmix, rope, o, lse, stream));
}

size_t maglev_swa_inject_bwd_workspace(const maglev_geom_t *g)
{
    Geom G;
    if (check_geom(g, &G) != MAGLEV_OK) return 0;
    BwdWorkspace layout;
    return bwd_workspace_bytes(G, &layout, nullptr, BwdKind::Sigma);
}

maglev_status_t maglev_swa_inject_bwd(const maglev_geom_t *g, const void *q, const void *kmix,
                                      const void *vmix, const void *kmem, const void *vmem,
                                      const float *gate_logit, const void *o, const float *lse,
                                      const void *dO, const void *m_prime, const void *W_Km,
                                      const void *W_Vm, void *dq, void *dk, void *dv,
                                      float *dm_prime, float *dW_Km, float *dW_Vm, float *dgate,
                                      unsigned accumulate, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    if (G.N() == 0)   // no tokens: only the parameter gradients are written (as zeros)
        st = check_ptrs({W_Km, W_Vm, dW_Km, dW_Vm});
    else
        st = check_ptrs({q, kmix, vmix, kmem, vmem, o, lse, dO, m_prime, W_Km, W_Vm, dq, dk, dv,
                         dm_prime, dW_Km, dW_Vm});
    if (st != MAGLEV_OK) return st;
    if (!gate_logit || !dgate) return fail(MAGLEV_ERR_INVALID_VALUE, "gate_logit or dgate is NULL");
    if (accumulate & ~7u) return fail(MAGLEV_ERR_INVALID_VALUE, "unknown accumulate bits");
    BwdWorkspace layout;
    const size_t need = bwd_workspace_bytes(G, &layout, static_cast<char *>(workspace), BwdKind::Sigma);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(MAGLEV_ERR_WORKSPACE, "workspace missing or too small");
    if (workspace && !aligned16(workspace))
        return fail(MAGLEV_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    const float2 *rope = nullptr;
    st = table_for(G, stream, &rope);
    if (st != MAGLEV_OK) return st;
    return launched(stream, launch_bwd(G, q, kmix, vmix, kmem, vmem, gate_logit, o, lse, dO, m_prime, W_Km,
                                 W_Vm, dq, dk, dv, dm_prime, dW_Km, dW_Vm, dgate, accumulate,
                                 layout, rope, stream));
}

size_t maglev_consistency_loss_workspace(int64_t N, int32_t d)
{
    if (N < 0 || d < 8 || (d % 8) != 0) return 0;
    return loss_workspace_bytes(N, d);
}

static maglev_status_t check_loss_args(int64_t N, int32_t d, float lambda, int32_t dtype,
                                       const void *m, const void *m_prime, const float *loss,
                                       const float *dm, const float *dm_prime,
                                       unsigned accumulate)
{
    if (N < 0) return fail(MAGLEV_ERR_INVALID_VALUE, "N must be >= 0");
    if (d < 8 || (d % 8) != 0) return fail(MAGLEV_ERR_INVALID_VALUE, "d must be a positive multiple of 8");
    if (!(lambda == lambda)) return fail(MAGLEV_ERR_INVALID_VALUE, "lambda is NaN");
    maglev_status_t st = check_dtype(dtype);
    if (st != MAGLEV_OK) return st;
    if (N > 0) {   // N == 0: the loss is 0 and nothing else is touched
        st = check_ptrs({m, m_prime});
        if (st != MAGLEV_OK) return st;
    }
    if (!loss) return fail(MAGLEV_ERR_INVALID_VALUE, "loss is NULL");
    if ((dm && !aligned16(dm)) || (dm_prime && !aligned16(dm_prime)))
        return fail(MAGLEV_ERR_MISALIGNED, "dm / dm_prime not 16-byte aligned");
    if (accumulate & ~7u) return fail(MAGLEV_ERR_INVALID_VALUE, "unknown accumulate bits");
    return MAGLEV_OK;
}

maglev_status_t maglev_consistency_loss(int64_t N, int32_t d, float lambda, int32_t dtype,
                                        const void *m, const void *m_prime, float *loss,
                                        float *dm, float *dm_prime, unsigned accumulate,
                                        void *workspace, size_t workspace_bytes,
                                        hipStream_t stream)
{
    maglev_status_t st =
        check_loss_args(N, d, lambda, dtype, m, m_prime, loss, dm, dm_prime, accumulate);
    if (st != MAGLEV_OK) return st;
    const size_t need = loss_workspace_bytes(N, d);
    if (!workspace || workspace_bytes < need)
        return fail(MAGLEV_ERR_WORKSPACE, "workspace missing or too small");
    if (!aligned16(workspace)) return fail(MAGLEV_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    return launched(stream, launch_loss(N, d, lambda, dtype, m, m_prime, loss, dm, dm_prime, accumulate,
                                  workspace, stream));
}

maglev_status_t maglev_consistency_loss_noalloc(int64_t N, int32_t d, float lambda,
                                                int32_t dtype, const void *m,
                                                const void *m_prime, float *loss, float *dm,
                                                float *dm_prime, unsigned accumulate,
                                                hipStream_t stream)
{
    maglev_status_t st =
        check_loss_args(N, d, lambda, dtype, m, m_prime, loss, dm, dm_prime, accumulate);
    if (st != MAGLEV_OK) return st;
    if (loss_workspace_bytes(N, d) > loss_scratch_bytes())
        return fail(MAGLEV_ERR_UNSUPPORTED, "the partial sums exceed the library's device scratch");
    float *scr = nullptr;
    st = hip_status(loss_scratch_address(&scr));
    if (st != MAGLEV_OK) return st;
    return launched(stream, launch_loss(N, d, lambda, dtype, m, m_prime, loss, dm, dm_prime, accumulate,
                                  scr, stream));
}

static bool head_sizes_ok(int64_t N, int32_t d, int64_t V)
{
    return N >= 1 && N <= INT32_MAX && d >= 16 && (d % 16) == 0 && V >= 16 && (V % 8) == 0 &&
           V <= INT32_MAX;
}

size_t maglev_lm_head_workspace(int64_t N, int32_t d, int64_t V, int32_t dtype)
{
    if (!head_sizes_ok(N, d, V) || (dtype != MAGLEV_F32 && dtype != MAGLEV_BF16)) return 0;
    HeadWorkspace L;
    return lm_head_workspace_bytes(N, d, V, dtype, &L, nullptr);
}

maglev_status_t maglev_lm_head(int64_t N, int32_t d, int64_t V, float cap, float eps,
                               float lambda, int32_t dtype, const void *h, const void *U,
                               const int64_t *targets, const void *m_prime, void *m, float *loss,
                               float *dh, float *dU, unsigned accumulate, void *workspace,
                               size_t workspace_bytes, hipStream_t stream)
{
    if (!head_sizes_ok(N, d, V))
        return fail(MAGLEV_ERR_INVALID_VALUE,
                    "need N >= 1, d a multiple of 16, V a multiple of 8 and >= 16");
    if (!(cap > 0.0f && cap <= 64.0f)) return fail(MAGLEV_ERR_INVALID_VALUE, "cap must be in (0, 64]");
    if (!(eps >= 0.0f) || !isfinite(eps)) return fail(MAGLEV_ERR_INVALID_VALUE, "eps must be finite and >= 0");
    if (!(lambda == lambda)) return fail(MAGLEV_ERR_INVALID_VALUE, "lambda is NaN");
    maglev_status_t st = check_dtype(dtype);
    if (st != MAGLEV_OK) return st;
    st = check_ptrs({h, U, m});
    if (st != MAGLEV_OK) return st;
    if (!targets) return fail(MAGLEV_ERR_INVALID_VALUE, "targets is NULL");
    if (!loss) return fail(MAGLEV_ERR_INVALID_VALUE, "loss is NULL");
    if ((m_prime && !aligned16(m_prime)) || (dh && !aligned16(dh)) || (dU && !aligned16(dU)))
        return fail(MAGLEV_ERR_MISALIGNED, "m_prime / dh / dU not 16-byte aligned");
    if (accumulate & ~7u) return fail(MAGLEV_ERR_INVALID_VALUE, "unknown accumulate bits");
    HeadWorkspace L;
    const size_t need = lm_head_workspace_bytes(N, d, V, dtype, &L, nullptr);
    if (!workspace || workspace_bytes < need)
        return fail(MAGLEV_ERR_WORKSPACE, "workspace missing or too small");
    if (!aligned16(workspace)) return fail(MAGLEV_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    lm_head_workspace_bytes(N, d, V, dtype, &L, static_cast<char *>(workspace));
    return launched(stream, launch_lm_head(N, d, V, cap, eps, lambda, dtype, h, U, targets, m_prime, m,
                                     loss, dh, dU, accumulate, L, stream));
}

size_t maglev_decode_workspace(int32_t Bs, int32_t H, int32_t Dh, int32_t W)
{
    if (Bs < 0 || H < 1 || (Dh != 64 && Dh != 128) || W < 1) return 0;
    return decode_workspace_bytes(Bs, H, Dh, W);
}

maglev_status_t maglev_decode_step(int32_t Bs, int32_t H, int32_t Dh, int32_t W,
                                   float rope_base, float scale, int32_t dtype, const void *q,
                                   const void *k, const void *v, const void *kmem,
                                   const void *vmem, int64_t mem_stride,
                                   const float *gate_logit, void *kcache, void *vcache,
                                   const int64_t *pos, void *o, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream)
{
    if (Bs < 0 || H < 1 || W < 1) return fail(MAGLEV_ERR_INVALID_VALUE, "need Bs >= 0, H >= 1, W >= 1");
    if (Dh != 64 && Dh != 128) return fail(MAGLEV_ERR_UNSUPPORTED, "Dh must be 64 or 128");
    if (!(scale == scale) || !(rope_base == rope_base))
        return fail(MAGLEV_ERR_INVALID_VALUE, "scale and rope_base must not be NaN");
    maglev_status_t st = check_dtype(dtype);
    if (st != MAGLEV_OK) return st;
    if (mem_stride == 0) mem_stride = (int64_t)H * Dh;
    if (mem_stride < (int64_t)H * Dh || mem_stride % 8 != 0)
        return fail(MAGLEV_ERR_INVALID_VALUE, "mem_stride must be 0 or a multiple of 8 >= H*Dh");
    if (Bs == 0) return MAGLEV_OK;   // no streams
    st = check_ptrs({q, k, v, kmem, vmem, kcache, vcache, o});
    if (st != MAGLEV_OK) return st;
    if (!gate_logit || !pos) return fail(MAGLEV_ERR_INVALID_VALUE, "gate_logit or pos is NULL");
    if ((double)Bs * H * W * Dh > 4.0e12) return fail(MAGLEV_ERR_INVALID_VALUE, "ring too large");
    if ((int64_t)Bs * H > 2147483647) return fail(MAGLEV_ERR_INVALID_VALUE, "Bs*H must be below 2^31");
    const size_t need = decode_workspace_bytes(Bs, H, Dh, W);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(MAGLEV_ERR_WORKSPACE, "workspace missing or too small");
    if (workspace && !aligned16(workspace))
        return fail(MAGLEV_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    const float sc = scale > 0.0f ? scale : (float)(1.0 / sqrt((double)Dh));
    return launched(stream, launch_decode(Bs, H, Dh, W, rope_base, sc, dtype, q, k, v, kmem, vmem,
                                    mem_stride, gate_logit, nullptr, 0.0f, kcache, vcache, pos, o,
                                    workspace, stream));
}

// ---- gated mixing form --------------------------------------------------------

namespace {
maglev_status_t check_gated(const Geom &G, const float *gates, float eps)
{
    if (G.HD() > 4096) return fail(MAGLEV_ERR_UNSUPPORTED, "gated form needs H*Dh <= 4096");
    if (!(eps >= 0.0f) || !(eps < INFINITY))
        return fail(MAGLEV_ERR_INVALID_VALUE, "eps must be finite and >= 0");
    if (!gates) return fail(MAGLEV_ERR_INVALID_VALUE, "gates is NULL");
    return MAGLEV_OK;
}
}  // namespace

maglev_status_t maglev_mem_project_gated(const maglev_geom_t *g, int shift, const void *m,
                                         const void *W_Km, const void *W_Vm, const void *k,
                                         const void *v, const float *gates, float eps,
                                         void *kproj, void *vmem, void *kmix, void *vmix,
                                         hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    if (shift != 0 && shift != 1) return fail(MAGLEV_ERR_INVALID_VALUE, "shift must be 0 or 1");
    st = check_gated(G, gates, eps);
    if (st != MAGLEV_OK) return st;
    if (G.N() == 0) return MAGLEV_OK;
    st = check_ptrs({m, W_Km, W_Vm, k, v, kproj, vmem, kmix, vmix});
    if (st != MAGLEV_OK) return st;
    const float2 *rope = nullptr;
    st = table_for(G, stream, &rope);
    if (st != MAGLEV_OK) return st;
    hipError_t e = launch_project(G, shift, m, W_Km, W_Vm, kproj, vmem, stream);
    if (e == hipSuccess)
        e = launch_gated_mix(G, k, v, kproj, vmem, gates, eps, rope, kmix, vmix, stream);
    return launched(stream, e);
}

size_t maglev_swa_inject_bwd_gated_workspace(const maglev_geom_t *g)
{
    Geom G;
    if (check_geom(g, &G) != MAGLEV_OK || G.HD() > 4096) return 0;
    BwdWorkspace layout;
    return bwd_workspace_bytes(G, &layout, nullptr, BwdKind::Gated);
}

maglev_status_t maglev_swa_inject_bwd_gated(
    const maglev_geom_t *g, const void *q, const void *kmix, const void *vmix, const void *k,
    const void *v, const void *kproj, const void *vmem, const float *gates, float eps,
    const void *o, const float *lse, const void *dO, const void *m_prime, const void *W_Km,
    const void *W_Vm, void *dq, void *dk, void *dv, float *dm_prime, float *dW_Km, float *dW_Vm,
    float *dgates, unsigned accumulate, void *workspace, size_t workspace_bytes,
    hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    st = check_gated(G, gates, eps);
    if (st != MAGLEV_OK) return st;
    if (G.N() == 0)
        st = check_ptrs({W_Km, W_Vm, dW_Km, dW_Vm});
    else
        st = check_ptrs({q, kmix, vmix, k, v, kproj, vmem, o, lse, dO, m_prime, W_Km, W_Vm, dq,
                         dk, dv, dm_prime, dW_Km, dW_Vm});
    if (st != MAGLEV_OK) return st;
    if (!dgates) return fail(MAGLEV_ERR_INVALID_VALUE, "dgates is NULL");
    if (accumulate & ~7u) return fail(MAGLEV_ERR_INVALID_VALUE, "unknown accumulate bits");
    BwdWorkspace layout;
    const size_t need = bwd_workspace_bytes(G, &layout, static_cast<char *>(workspace), BwdKind::Gated);
    if (G.N() > 0 && (!workspace || workspace_bytes < need))
        return fail(MAGLEV_ERR_WORKSPACE, "workspace missing or too small");
    if (workspace && !aligned16(workspace))
        return fail(MAGLEV_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    const float2 *rope = nullptr;
    st = table_for(G, stream, &rope);
    if (st != MAGLEV_OK) return st;
    return launched(stream, launch_bwd_gated(G, q, kmix, vmix, k, v, kproj, vmem, gates, eps, o, lse, dO,
                                       m_prime, W_Km, W_Vm, dq, dk, dv, dm_prime, dW_Km, dW_Vm,
                                       dgates, accumulate, layout, rope, stream));
}

maglev_status_t maglev_decode_step_gated(int32_t Bs, int32_t H, int32_t Dh, int32_t W,
                                         float rope_base, float scale, int32_t dtype,
                                         const void *q, const void *k, const void *v,
                                         const void *kproj, const void *vmem, int64_t mem_stride,
                                         const float *gates, float eps, void *kcache,
                                         void *vcache, const int64_t *pos, void *o,
                                         void *workspace, size_t workspace_bytes,
                                         hipStream_t stream)
{
    if (Bs < 0 || H < 1 || W < 1) return fail(MAGLEV_ERR_INVALID_VALUE, "need Bs >= 0, H >= 1, W >= 1");
    if (Dh != 64 && Dh != 128) return fail(MAGLEV_ERR_UNSUPPORTED, "Dh must be 64 or 128");
    if (!(scale == scale) || !(rope_base == rope_base))
        return fail(MAGLEV_ERR_INVALID_VALUE, "scale and rope_base must not be NaN");
    if (!(eps >= 0.0f) || !(eps < INFINITY))
        return fail(MAGLEV_ERR_INVALID_VALUE, "eps must be finite and >= 0");
    maglev_status_t st = check_dtype(dtype);
    if (st != MAGLEV_OK) return st;
    if (mem_stride == 0) mem_stride = (int64_t)H * Dh;
    if (mem_stride < (int64_t)H * Dh || mem_stride % 8 != 0)
        return fail(MAGLEV_ERR_INVALID_VALUE, "mem_stride must be 0 or a multiple of 8 >= H*Dh");
    if (Bs == 0) return MAGLEV_OK;
    st = check_ptrs({q, k, v, kproj, vmem, kcache, vcache, o});
    if (st != MAGLEV_OK) return st;
    if (!gates || !pos) return fail(MAGLEV_ERR_INVALID_VALUE, "gates or pos is NULL");
    if ((double)Bs * H * W * Dh > 4.0e12) return fail(MAGLEV_ERR_INVALID_VALUE, "ring too large");
    if ((int64_t)Bs * H > 2147483647) return fail(MAGLEV_ERR_INVALID_VALUE, "Bs*H must be below 2^31");
    const size_t need = decode_workspace_bytes(Bs, H, Dh, W);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(MAGLEV_ERR_WORKSPACE, "workspace missing or too small");
    if (workspace && !aligned16(workspace))
        return fail(MAGLEV_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    const float sc = scale > 0.0f ? scale : (float)(1.0 / sqrt((double)Dh));
    return launched(stream, launch_decode(Bs, H, Dh, W, rope_base, sc, dtype, q, k, v, kproj, vmem,
                                    mem_stride, nullptr, gates, eps, kcache, vcache, pos, o,
                                    workspace, stream));
}

// ---- attention without injection ---------------------------------------------

maglev_status_t maglev_rope_keys(const maglev_geom_t *g, const void *k, void *krot,
                                 hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    if (G.N() == 0) return MAGLEV_OK;
    st = check_ptrs({k, krot});
    if (st != MAGLEV_OK) return st;
    if (k == krot) return fail(MAGLEV_ERR_INVALID_VALUE, "krot must not alias k");
    const float2 *rope = nullptr;
    st = table_for(G, stream, &rope);
    if (st != MAGLEV_OK) return st;
    return launched(stream, launch_rope_keys(G, k, rope, krot, stream));
}

size_t maglev_attn_bwd_workspace(const maglev_geom_t *g)
{
    Geom G;
    if (check_geom(g, &G) != MAGLEV_OK) return 0;
    BwdWorkspace layout;
    return bwd_workspace_bytes(G, &layout, nullptr, BwdKind::Attn);
}

maglev_status_t maglev_attn_bwd(const maglev_geom_t *g, const void *q, const void *krot,
                                const void *v, const void *o, const float *lse, const void *dO,
                                void *dq, void *dk, void *dv, void *workspace,
                                size_t workspace_bytes, hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    if (G.N() == 0) return MAGLEV_OK;
    st = check_ptrs({q, krot, v, o, lse, dO, dq, dk, dv});
    if (st != MAGLEV_OK) return st;
    BwdWorkspace layout;
    const size_t need = bwd_workspace_bytes(G, &layout, static_cast<char *>(workspace), BwdKind::Attn);
    if (!workspace || workspace_bytes < need)
        return fail(MAGLEV_ERR_WORKSPACE, "workspace missing or too small");
    if (!aligned16(workspace)) return fail(MAGLEV_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    const float2 *rope = nullptr;
    st = table_for(G, stream, &rope);
    if (st != MAGLEV_OK) return st;
    return launched(stream, launch_attn_bwd(G, q, krot, v, o, lse, dO, dq, dk, dv, layout, rope, stream));
}

// ---- layers sharing one memory projection ---------------------------------------

maglev_status_t maglev_mix_entries(const maglev_geom_t *g, const void *k, const void *v,
                                   const void *kmem, const void *vmem, const float *gate_logit,
                                   void *kmix, void *vmix, hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    if (G.N() == 0) return MAGLEV_OK;
    st = check_ptrs({k, v, kmem, vmem, kmix, vmix});
    if (st != MAGLEV_OK) return st;
    if (!gate_logit) return fail(MAGLEV_ERR_INVALID_VALUE, "gate_logit is NULL");
    const float2 *rope = nullptr;
    st = table_for(G, stream, &rope);
    if (st != MAGLEV_OK) return st;
    return launched(stream, launch_mix(G, k, v, kmem, vmem, gate_logit, rope, kmix, vmix, stream));
}

size_t maglev_swa_inject_bwd_shared_workspace(const maglev_geom_t *g)
{
    Geom G;
    if (check_geom(g, &G) != MAGLEV_OK) return 0;
    BwdWorkspace layout;
    return bwd_workspace_bytes(G, &layout, nullptr, BwdKind::Shared);
}

maglev_status_t maglev_swa_inject_bwd_shared(const maglev_geom_t *g, const void *q,
                                             const void *kmix, const void *vmix,
                                             const void *kmem, const void *vmem,
                                             const float *gate_logit, const void *o,
                                             const float *lse, const void *dO, void *dq,
                                             void *dk, void *dv, float *dkmem, float *dvmem,
                                             float *dgate, unsigned accumulate, void *workspace,
                                             size_t workspace_bytes, hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    if (!gate_logit || !dgate) return fail(MAGLEV_ERR_INVALID_VALUE, "gate_logit or dgate is NULL");
    if (accumulate & ~5u) return fail(MAGLEV_ERR_INVALID_VALUE, "unknown accumulate bits");
    if (G.N() > 0) {
        st = check_ptrs({q, kmix, vmix, kmem, vmem, o, lse, dO, dq, dk, dv, dkmem, dvmem});
        if (st != MAGLEV_OK) return st;
    }
    BwdWorkspace layout;
    const size_t need = bwd_workspace_bytes(G, &layout, static_cast<char *>(workspace), BwdKind::Shared);
    if (G.N() > 0 && (!workspace || workspace_bytes < need))
        return fail(MAGLEV_ERR_WORKSPACE, "workspace missing or too small");
    if (workspace && !aligned16(workspace))
        return fail(MAGLEV_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    const float2 *rope = nullptr;
    if (G.N() > 0) {
        st = table_for(G, stream, &rope);
        if (st != MAGLEV_OK) return st;
    }
    return launched(stream, launch_bwd_shared(G, q, kmix, vmix, kmem, vmem, gate_logit, o, lse, dO, dq,
                                        dk, dv, dkmem, dvmem, dgate, accumulate, layout, rope,
                                        stream));
}

maglev_status_t maglev_mix_entries_gated(const maglev_geom_t *g, const void *k, const void *v,
                                         const void *kproj, const void *vmem, const float *gates,
                                         float eps, void *kmix, void *vmix, hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    st = check_gated(G, gates, eps);
    if (st != MAGLEV_OK) return st;
    if (G.N() == 0) return MAGLEV_OK;
    st = check_ptrs({k, v, kproj, vmem, kmix, vmix});
    if (st != MAGLEV_OK) return st;
    const float2 *rope = nullptr;
    st = table_for(G, stream, &rope);
    if (st != MAGLEV_OK) return st;
    return launched(stream, launch_gated_mix(G, k, v, kproj, vmem, gates, eps, rope, kmix, vmix, stream));
}

size_t maglev_swa_inject_bwd_shared_gated_workspace(const maglev_geom_t *g)
{
    Geom G;
    if (check_geom(g, &G) != MAGLEV_OK || G.HD() > 4096) return 0;
    BwdWorkspace layout;
    return bwd_workspace_bytes(G, &layout, nullptr, BwdKind::SharedGated);
}

maglev_status_t maglev_swa_inject_bwd_shared_gated(
    const maglev_geom_t *g, const void *q, const void *kmix, const void *vmix, const void *k,
    const void *v, const void *kproj, const void *vmem, const float *gates, float eps,
    const void *o, const float *lse, const void *dO, void *dq, void *dk, void *dv, float *dkproj,
    float *dvmem, float *dgates, unsigned accumulate, void *workspace, size_t workspace_bytes,
    hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    st = check_gated(G, gates, eps);
    if (st != MAGLEV_OK) return st;
    if (!dgates) return fail(MAGLEV_ERR_INVALID_VALUE, "dgates is NULL");
    if (accumulate & ~5u) return fail(MAGLEV_ERR_INVALID_VALUE, "unknown accumulate bits");
    if (G.N() > 0) {
        st = check_ptrs({q, kmix, vmix, k, v, kproj, vmem, o, lse, dO, dq, dk, dv, dkproj, dvmem});
        if (st != MAGLEV_OK) return st;
    }
    BwdWorkspace layout;
    const size_t need =
        bwd_workspace_bytes(G, &layout, static_cast<char *>(workspace), BwdKind::SharedGated);
    if (G.N() > 0 && (!workspace || workspace_bytes < need))
        return fail(MAGLEV_ERR_WORKSPACE, "workspace missing or too small");
    if (workspace && !aligned16(workspace))
        return fail(MAGLEV_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    const float2 *rope = nullptr;
    if (G.N() > 0) {
        st = table_for(G, stream, &rope);
        if (st != MAGLEV_OK) return st;
    }
    return launched(stream, launch_bwd_shared_gated(G, q, kmix, vmix, k, v, kproj, vmem, gates, eps, o,
                                              lse, dO, dq, dk, dv, dkproj, dvmem, dgates,
                                              accumulate, layout, rope, stream));
}

size_t maglev_mem_project_bwd_workspace(const maglev_geom_t *g)
{
    Geom G;
    if (check_geom(g, &G) != MAGLEV_OK) return 0;
    BwdWorkspace layout;
    return bwd_workspace_bytes(G, &layout, nullptr, BwdKind::Proj);
}

maglev_status_t maglev_mem_project_bwd(const maglev_geom_t *g, const float *dkmem,
                                       const float *dvmem, const void *m_prime, const void *W_Km,
                                       const void *W_Vm, float *dm_prime, float *dW_Km,
                                       float *dW_Vm, unsigned accumulate, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream)
{
    Geom G;
    maglev_status_t st = check_geom(g, &G);
    if (st != MAGLEV_OK) return st;
    if (accumulate & ~3u) return fail(MAGLEV_ERR_INVALID_VALUE, "unknown accumulate bits");
    if (G.N() == 0)
        st = check_ptrs({W_Km, W_Vm, dW_Km, dW_Vm});
    else
        st = check_ptrs({dkmem, dvmem, m_prime, W_Km, W_Vm, dm_prime, dW_Km, dW_Vm});
    if (st != MAGLEV_OK) return st;
    BwdWorkspace layout;
    const size_t need = bwd_workspace_bytes(G, &layout, static_cast<char *>(workspace), BwdKind::Proj);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(MAGLEV_ERR_WORKSPACE, "workspace missing or too small");
    if (workspace && !aligned16(workspace))
        return fail(MAGLEV_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    return launched(stream, launch_mem_project_bwd(G, dkmem, dvmem, m_prime, W_Km, W_Vm, dm_prime, dW_Km,
                                             dW_Vm, accumulate, layout, stream));
}

maglev_status_t maglev_decode_advance(int32_t Bs, int64_t *pos, hipStream_t stream)
{
    if (Bs < 0) return fail(MAGLEV_ERR_INVALID_VALUE, "Bs must be >= 0");
    if (!pos) return fail(MAGLEV_ERR_INVALID_VALUE, "pos is NULL");
    if (Bs == 0) return MAGLEV_OK;
    return launched(stream, launch_advance(Bs, pos, stream));
}

}  // extern "C"
