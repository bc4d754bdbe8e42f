// internal.hpp -- host-side declarations shared by the C-ABI layer and the
// kernel translation units. Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "maglev.h"

namespace maglev {

// Validated geometry handed to launchers (mirrors maglev_geom_t).
struct Geom {
    int64_t B, T;
    int H, Dh, d, W;
    int64_t pos0;
    float rope_base;
    float scale;   // resolved: > 0
    int dtype;     // maglev_dtype_t
    int64_t N() const { return B * T; }
    int HD() const { return H * Dh; }
};

// RoPE table: float2 (cos, sin) [max_pos][Dh/2] for (device, Dh, base), or
// nullptr when base <= 0. Grows on demand (synchronous upload).
maglev_status_t rope_table(int Dh, float base, int64_t max_pos, const float2 **table);

// ---- memory projection: out rows (b,t) = in(b, t - shift) * W^T ----------
hipError_t launch_project(const Geom &g, int shift, const void *m, const void *W_Km,
                          const void *W_Vm, void *kmem, void *vmem, hipStream_t s);

// ---- gated mix of the memory terms into the local K/V entries -----------------
//   kmix = R (k + s_h kmem), vmix = v + s_h vmem   (R linear: R k + s R kmem)
hipError_t launch_mix(const Geom &g, const void *k, const void *v, const void *kmem,
                      const void *vmem, const float *gate, const float2 *rope, void *kmix,
                      void *vmix, hipStream_t s);

// ---- attention forward -----------------------------------------------------
hipError_t launch_attn_fwd(const Geom &g, const void *q, const void *kmix, const void *vmix,
                           const float2 *rope, void *o, float *lse, hipStream_t s);

// ---- backward --------------------------------------------------------------
struct BwdWorkspace {
    float *D;            // [B,H,T]  rowsum(dO * O) (float32 path)
    float *ds_part;      // [B,H,T] per-key d loss / d s_h terms (float32 path)
    float *rowdot;       // [2*H*Dh] <W[r,:], G[r,:]> per weight row (bf16 path)
    void *W_scaled;      // [d, 2*H*Dh] dtype: (s_h * [W_Km; W_Vm])^T (rows scaled, then transposed)
    float *dW_part;      // [ksplit, 2*H*Dh, d] split-K partials (may be unused)
    void *q_rot;         // [B,T,H,Dh] dtype: rotated queries (bf16 path)
    float *lse2;         // [B*H, Tp] lse * log2(e), zero beyond T (bf16 path)
    float *Dp;           // [B*H, Tp] rowsum(dO * O), zero beyond T (bf16 path)
    int64_t Tp;          // T rounded up to a multiple of 32
    int ksplit;
    int n_key_tiles;
    // bf16 path, Dh = 128: dS = P (dP - D) of every in-band 32 x 32 tile as the
    // dK/dV pass rounded it for its dK product, [B*H][nt32][ds_tiles][32 k][32 q],
    // tile (kt, j) covering keys 32 kt.. and queries 32 (kt + j)..; the dQ pass
    // reads it instead of recomputing the scores (null: dQ recomputes).
    void *ds;
    int nt32;            // ceil(T / 32)
    int ds_tiles;        // query tiles stored per key tile

    // gated form only
    void *dkp;           // [B,T,H*Dh] dtype: d loss / d (W_Km m'), before the norm
    void *dvm;           // [B,T,H*Dh] dtype: d loss / d (W_Vm m')
    float *gpart;        // [g_blocks][4][H*Dh] per-workgroup gate partial sums
    int g_rows, g_blocks;
};
// Which backward the workspace serves: the sigma-gated layer path, the gated
// layer path, or attention alone (no memory term, no projection).
// Shared: one layer of a stack sharing a projection (attention backward and
// the memory-gradient accumulation); SharedGated: the same for the gated mix;
// Proj: that projection's backward alone.
enum class BwdKind { Sigma, Gated, Attn, Shared, SharedGated, Proj };
constexpr int kSharedTokens = 128;   // tokens per workgroup of the shared accumulation
size_t bwd_workspace_bytes(const Geom &g, BwdWorkspace *layout, char *base, BwdKind kind);

hipError_t launch_bwd(const Geom &g, const void *q, const void *kmix, const void *vmix,
                      const void *kmem, const void *vmem, const float *gate, const void *o,
                      const float *lse, const void *dO, const void *m_prime, const void *W_Km,
                      const void *W_Vm, void *dq, void *dk, void *dv, float *dm_prime,
                      float *dW_Km, float *dW_Vm, float *dgate, unsigned accumulate,
                      const BwdWorkspace &ws, const float2 *rope, hipStream_t s);

// ---- gated form: k~ = g_kl R k + g_kr R RMSNorm(kp), v~ = g_vl v + g_vr vm ----
// gates [4][H*Dh] float32 logits (a_kl, a_kr, a_vl, a_vr), g = 2 sigmoid(a).
void gated_partition(int64_t N, int *rows_per_block, int *blocks);
hipError_t launch_gated_mix(const Geom &g, const void *k, const void *v, const void *kproj,
                            const void *vmem, const float *gates, float eps, const float2 *rope,
                            void *kmix, void *vmix, hipStream_t s);
// dk/dv: in = gradients of the mixed entries, out = gradients of k and v.
// The projection gradients go to ws.dkp/ws.dvm (dtype), or with dkp32 != null
// to the float32 dkp32/dvm32 (accumulate bit 0: added).
hipError_t launch_gated_mix_bwd(const Geom &g, const void *k, const void *v, const void *kproj,
                                const void *vmem, const float *gates, float eps,
                                const float2 *rope, void *dk, void *dv, const BwdWorkspace &ws,
                                float *dgates, unsigned accumulate, float *dkp32, float *dvm32,
                                hipStream_t s);
hipError_t launch_bwd_gated(const Geom &g, const void *q, const void *kmix, const void *vmix,
                            const void *k, const void *v, const void *kproj, const void *vmem,
                            const float *gates, float eps, const void *o, const float *lse,
                            const void *dO, const void *m_prime, const void *W_Km,
                            const void *W_Vm, void *dq, void *dk, void *dv, float *dm_prime,
                            float *dW_Km, float *dW_Vm, float *dgates, unsigned accumulate,
                            const BwdWorkspace &ws, const float2 *rope, hipStream_t s);

// ---- attention without injection (the prefiller's layers) ------------------
// kr = R_{pos0+t} k; the backward gives dq, dk (w.r.t. the unrotated k), dv.
hipError_t launch_rope_keys(const Geom &g, const void *k, const float2 *rope, void *kr,
                            hipStream_t s);
hipError_t launch_attn_bwd(const Geom &g, const void *q, const void *kr, const void *v,
                           const void *o, const float *lse, const void *dO, void *dq, void *dk,
                           void *dv, const BwdWorkspace &ws, const float2 *rope, hipStream_t s);

// ---- layers sharing one memory projection ------------------------------------
// Per layer: attention backward (dq, dk, dv) and dkm (+)= s dk, dvm (+)= s dv
// (float32), dgate (+)= s(1-s) sum <kmem, dk> + <vmem, dv>. accumulate bit 0:
// dkm/dvm +=, bit 2: dgate +=.
hipError_t launch_bwd_shared(const Geom &g, const void *q, const void *kmix, const void *vmix,
                             const void *kmem, const void *vmem, const float *gate,
                             const void *o, const float *lse, const void *dO, void *dq,
                             void *dk, void *dv, float *dkmem, float *dvmem, float *dgate,
                             unsigned accumulate, const BwdWorkspace &ws, const float2 *rope,
                             hipStream_t s);
// Gated form over a shared projection, per layer: attention backward, the
// gated mix backward (dk, dv of the local features, dgates), and the layer's
// share of the gradients of the shared pre-norm projections kp, vm into the
// float32 dkp, dvm (accumulate bit 0: added; bit 2: dgates added).
hipError_t launch_bwd_shared_gated(const Geom &g, const void *q, const void *kmix,
                                   const void *vmix, const void *k, const void *v,
                                   const void *kproj, const void *vmem, const float *gates,
                                   float eps, const void *o, const float *lse, const void *dO,
                                   void *dq, void *dk, void *dv, float *dkp, float *dvm,
                                   float *dgates, unsigned accumulate, const BwdWorkspace &ws,
                                   const float2 *rope, hipStream_t s);
// Once per pass: dm' and dW from the summed float32 memory gradients.
hipError_t launch_mem_project_bwd(const Geom &g, const float *dkmem, const float *dvmem,
                                  const void *m_prime, const void *W_Km, const void *W_Vm,
                                  float *dm_prime, float *dW_Km, float *dW_Vm, unsigned accumulate,
                                  const BwdWorkspace &ws, hipStream_t s);

// ---- consistency loss -------------------------------------------------------
size_t loss_workspace_bytes(int64_t N, int d);
hipError_t launch_loss(int64_t N, int d, float lambda, int dtype, const void *m,
                       const void *mp, float *loss, float *dm, float *dmp, unsigned accumulate,
                       void *ws, hipStream_t s);
// The allocation-free variant's partial sums: a device array of
// loss_scratch_bytes() bytes per GPU; its address on the current device
// (looked up on the first call per device).
size_t loss_scratch_bytes();
hipError_t loss_scratch_address(float **addr);

// ---- loss head -----------------------------------------------------------
struct HeadWorkspace {
    float *rstd = nullptr;     // [N] 1 / rms of each row of h
    float *ce = nullptr;       // [N] per-position cross-entropy
    float *logits = nullptr;   // [N, V] capped logits
    float *rowsum = nullptr;   // [N, column tiles] partial sums of exp(logit)
    void *dz = nullptr;        // [N, V] dtype, gradient w.r.t. the raw logits
    float *dm = nullptr;       // [N, d] gradient w.r.t. m
    void *ut = nullptr;        // [d, V] bf16: U transposed for the dm product (bf16 path)
    void *loss_ws = nullptr;   // consistency-loss partial sums
};
// Bytes of workspace; with base != nullptr, also carves it into *L.
size_t lm_head_workspace_bytes(int64_t N, int d, int64_t V, int dtype, HeadWorkspace *L,
                               char *base);
hipError_t launch_lm_head(int64_t N, int d, int64_t V, float cap, float eps, float lambda,
                          int dtype, const void *h, const void *U, const int64_t *targets,
                          const void *m_prime, void *m, float *loss, float *dh, float *dU,
                          unsigned acc, const HeadWorkspace &ws, hipStream_t s);

// ---- decode -----------------------------------------------------------------
size_t decode_workspace_bytes(int Bs, int H, int Dh, int W);
// gates == nullptr: the sigma-gated form with gate [H]; otherwise the gated
// form with gates [4][H*Dh] and kmem = the pre-norm projection (gate unused).
hipError_t launch_decode(int Bs, int H, int Dh, int W, float rope_base, float scale, int dtype,
                         const void *q, const void *k, const void *v, const void *kmem,
                         const void *vmem, int64_t mem_stride, const float *gate,
                         const float *gates, float eps, void *kcache, void *vcache,
                         const int64_t *pos, void *o, void *ws, hipStream_t s);
hipError_t launch_advance(int Bs, int64_t *pos, hipStream_t s);

}  // namespace maglev
