/*
 * maglev.h -- C ABI of the MI355X (gfx950) library for the Maglev decoder-P
 * attention path: causal sliding-window attention with recurrent K/V
 * injection, its backward, the memory-consistency loss and the recurrent
 * decode step on a W-slot ring cache.
 *
 * Sources (web summaries of the preprint "Maglev: Sliding Recurrent Memory"):
 *   [R-bg]   paper.rainbus.top, "Maglev：滑动窗口循环记忆", section 前置知识
 *            (sliding-window attention over the W most recent tokens; KV cache;
 *            feature-consistency loss; RoPE on both the local and the injected
 *            key before mixing).
 *   [R-mot]  same page, section 研究动机 (interface p(x_{t+1}, m_t | x_{t-W+1:t},
 *            M_{t-1}); memory window of W entries; cache cost equal to SWA).
 *   [R-core] same page, section 核心方法 (decoder P is sliding-window only, W=512;
 *            the shifted memory goes through a shared projection into K/V
 *            features mixed into the existing cache entries; no extra slots).
 *   [R-step] same page, section 方法步骤详情 (P(x_{1:T}, m'_{0:T-1}) with m'_0 = 0;
 *            recurrent K/V features from W^rec m'_{t-1}; gated mix; attention
 *            over the W most recent mixed entries; loss
 *            1/|I| sum_t [CE + lambda ||m_t - m'_t||^2 / sqrt(d)]; recurrent
 *            inference m_t = P(x_{t-W+1:t}, M_{t-1})).
 *   [G-train] gist.science, "Technische Samenvatting: Maglev - Sliding Recurrent
 *            Memory", section Trainingsmechanisme: Lifted Parallel Training
 *            (two parallel passes replace the sequential unroll).
 *   [G-inf]  same page, section Inferentiemechanisme (K/V injection through
 *            learned projections and gates; bounded decode cost).
 *
 * Mixing form implemented (the pages leave it open; one summary prints a
 * gated variant with a local gate and a normalised memory key):
 *   kmem_j = W_Km m'_{j-1},  vmem_j = W_Vm m'_{j-1}   (m'_{-1} := 0)
 *   k~_j   = R_j k_j + s_h R_j kmem_j,   v~_j = v_j + s_h vmem_j,
 *   s_h    = sigmoid(gate_logit[h]), one float32 logit per head,
 *   O_i    = sum_{j = max(0, i-W+1)}^{i} softmax_j(scale <R_i q_i, k~_j>) v~_j.
 * The mixed entries k~, v~ are formed once per token by maglev_mem_project
 * and read by the attention forward and backward.
 * The gated form that [R-step] prints is available as well (the *_gated
 * calls below): channel-wise gates g = 2 sigmoid(a) on both the local and the
 * recurrent term, and an RMSNorm on the projected memory key.
 * R_p rotates channel pair (c, c + Dh/2) by angle p * base^(-2c/Dh) (p = pos0 + t).
 *
 * Common conventions
 *   - Layouts are row-major: activations [B,T,H,Dh] (the [B,T,d_model] tensor
 *     viewed per head), memories [B,T,d], projection weights [H*Dh, d]
 *     (the weight of a linear layer d -> H*Dh), lse [B,H,T], ring caches
 *     [Bs,H,W,Dh].
 *   - Every pointer is a DEVICE pointer unless stated, owned by the caller; the
 *     library never frees caller memory and keeps no pointer after a call.
 *   - All work is enqueued on `stream`; calls are asynchronous and do not
 *     synchronise. Device faults surface at the caller's next synchronisation.
 *   - Element dtype: MAGLEV_F32 (float) or MAGLEV_BF16 (bfloat16) for the
 *     activation tensors named "dtype" below; gate logits, lse, loss and every
 *     parameter gradient are float32. Arithmetic accumulates in float32.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error the call returns a status other than MAGLEV_OK and writes nothing.
 *   - A call with no rows (B*T == 0, Bs == 0, N == 0) returns MAGLEV_OK after
 *     the geometry check without reading its data pointers (empty tensors may
 *     be NULL); only the parameter gradients of the backward are still
 *     written (zeroed unless accumulating).
 *   - The library keeps one internal device table per (device, Dh, rope_base):
 *     float32 cos/sin of the RoPE angles, computed on the host in double
 *     precision. It is created or grown on first use (a synchronous upload);
 *     call maglev_prepare() before capturing a HIP graph.
 */
#ifndef MAGLEV_H
#define MAGLEV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAGLEV_ABI_VERSION 6

typedef enum {
    MAGLEV_OK = 0,
    MAGLEV_ERR_INVALID_VALUE = 1, /* bad shape, NULL pointer, bad enum */
    MAGLEV_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. Dh not in {64,128}) */
    MAGLEV_ERR_MISALIGNED = 3,    /* a pointer is not 16-byte aligned */
    MAGLEV_ERR_WORKSPACE = 4,     /* workspace NULL or smaller than the query says */
    MAGLEV_ERR_HIP = 5            /* a HIP runtime call or launch failed */
} maglev_status_t;

typedef enum { MAGLEV_F32 = 0, MAGLEV_BF16 = 1 } maglev_dtype_t;

/* Geometry of one attention layer call.
 *   B, T      batch and sequence length (T >= 1)
 *   H, Dh     heads and head width; Dh in {64, 128}, H*Dh <= 65536
 *             (else MAGLEV_ERR_UNSUPPORTED)
 *   d         width of the memory m (d_model); multiple of 16
 *   W         window: query i sees keys max(0, i-W+1) .. i (W >= 1)
 *   pos0      absolute position of t = 0 (RoPE angle uses pos0 + t), >= 0
 *   rope_base RoPE base (10000 for nanochat); <= 0 disables the rotation
 *   scale     softmax scale; <= 0 selects 1/sqrt(Dh)
 *   dtype     maglev_dtype_t of the activation tensors */
typedef struct {
    int64_t B, T;
    int32_t H, Dh, d, W;
    int64_t pos0;
    float rope_base;
    float scale;
    int32_t dtype;
} maglev_geom_t;

/* Memory projection with the one-step shift, and the gated mix of the
 * projected memory into each token's own K/V entry ([R-step]: P consumes
 * m'_{0:T-1} with m'_0 = 0; [R-core]: the shifted memory passes through a
 * shared projection into K/V features mixed into the existing entries;
 * [R-bg]: the injected key is rotated at the local key's position before
 * mixing).
 *   shift = 1: input row (b,t) is m[b,t-1], row (b,0) is zero;
 *   shift = 0: input row (b,t) is m[b,t] (decode injects m_{t-1} directly).
 *   m [B,T,d] dtype; W_Km, W_Vm [H*Dh, d] dtype;
 *   kmem, vmem [B,T,H,Dh] dtype, written: kmem = input W_Km^T, vmem = input W_Vm^T.
 * Mixing (all five of k, v, gate_logit, kmix, vmix non-NULL, or all NULL):
 *   k, v [B,T,H,Dh] dtype (the token's local key/value, before RoPE);
 *   gate_logit [H] float32;
 *   kmix, vmix [B,T,H,Dh] dtype, written:
 *     kmix = R_{pos0+t} k + s_h R_{pos0+t} kmem,  vmix = v + s_h vmem.
 * Uses g->B, T, H, Dh, d, pos0, rope_base, dtype. */
maglev_status_t maglev_mem_project(const maglev_geom_t *g, int shift, const void *m,
                                   const void *W_Km, const void *W_Vm, const void *k,
                                   const void *v, const float *gate_logit, void *kmem,
                                   void *vmem, void *kmix, void *vmix, hipStream_t stream);

/* Forward of the injected sliding-window attention ([R-bg], [R-core], [R-step]):
 * rotate q and attend over the W most recent mixed entries (fully masked key
 * tiles are skipped).
 *   q [B,T,H,Dh] dtype (before RoPE);
 *   kmix, vmix [B,T,H,Dh] dtype: the mixed entries written by maglev_mem_project;
 *   o [B,T,H,Dh] dtype, written;
 *   lse [B,H,T] float32, written (log-sum-exp of the scaled scores; may be NULL
 *   when no backward follows). */
maglev_status_t maglev_swa_inject_fwd(const maglev_geom_t *g, const void *q, const void *kmix,
                                      const void *vmix, void *o, float *lse, hipStream_t stream);

/* Bytes of device workspace maglev_swa_inject_bwd needs for this geometry
 * (0 on invalid geometry). */
size_t maglev_swa_inject_bwd_workspace(const maglev_geom_t *g);

/* Backward of the layer path: attention, mixing, shift and projection (the
 * chain rule through the forward above; [R-step], [G-train]).
 * Inputs: q; the mixed entries kmix, vmix and the memory terms kmem, vmem
 * written by maglev_mem_project; gate_logit; the forward's o and lse; the
 * upstream gradient dO [B,T,H,Dh] dtype; m_prime [B,T,d] dtype (UNshifted, as
 * given to maglev_mem_project with shift = 1); W_Km, W_Vm [H*Dh, d] dtype.
 * Outputs:
 *   dq, dk, dv [B,T,H,Dh] dtype (overwritten): gradients w.r.t. q, k, v;
 *   dm_prime [B,T,d] float32: gradient w.r.t. m'; row T-1 gets no injection
 *     gradient (it is never consumed);
 *   dW_Km, dW_Vm [H*Dh, d] float32; dgate [H] float32 (w.r.t. the logits).
 * accumulate: bit 0 -> dm_prime +=, bit 1 -> dW_Km/dW_Vm +=, bit 2 -> dgate +=;
 *   a clear bit overwrites.
 * workspace: device buffer of at least maglev_swa_inject_bwd_workspace(g)
 *   bytes, owned by the caller; contents are scratch on return.
 * The result is deterministic: no floating-point atomics are used. */
maglev_status_t maglev_swa_inject_bwd(const maglev_geom_t *g, const void *q, const void *kmix,
                                      const void *vmix, const void *kmem, const void *vmem,
                                      const float *gate_logit, const void *o, const float *lse,
                                      const void *dO, const void *m_prime, const void *W_Km,
                                      const void *W_Vm, void *dq, void *dk, void *dv,
                                      float *dm_prime, float *dW_Km, float *dW_Vm, float *dgate,
                                      unsigned accumulate, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace maglev_consistency_loss needs (0 on invalid sizes). */
size_t maglev_consistency_loss_workspace(int64_t N, int32_t d);

/* Memory-consistency loss ([R-core], [R-step]):
 *   loss = lambda / (N sqrt(d)) * sum_{n,e} (m - m')^2     (float32 scalar)
 *   dm = 2 lambda (m - m') / (N sqrt(d)),  dm_prime = -dm   (float32 [N,d])
 *   m, m_prime [N, d] dtype; loss: device float32 scalar (written, or += when
 *   accumulate bit 2 is set); dm / dm_prime may be NULL; accumulate bit 0 ->
 *   dm +=, bit 1 -> dm_prime +=. d must be a multiple of 8.
 * The reduction is two-stage and deterministic. */
maglev_status_t maglev_consistency_loss(int64_t N, int32_t d, float lambda, int32_t dtype,
                                        const void *m, const void *m_prime, float *loss,
                                        float *dm, float *dm_prime, unsigned accumulate,
                                        void *workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* The consistency loss above for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving or training loops, harnesses
 * that forbid allocation): the same kernels and the same result bits, with
 * the partial sums in a device array of the library (2048 floats, 8 KB per
 * GPU, held until the process ends) instead of a workspace. Arguments and
 * accumulate bits as maglev_consistency_loss; nothing is allocated or freed.
 * The scratch holds the partial sums of every (N, d) (the grid is capped at
 * 2048 workgroups); a size whose partials would not fit returns
 * MAGLEV_ERR_UNSUPPORTED. The array's address is looked up on the first call
 * on a device (maglev_prepare does it ahead of capture). Every call on one
 * GPU shares the array: calls that overlap in time on one GPU race, so
 * serialise them (one stream, or events). */
maglev_status_t maglev_consistency_loss_noalloc(int64_t N, int32_t d, float lambda, int32_t dtype,
                                                const void *m, const void *m_prime, float *loss,
                                                float *dm, float *dm_prime, unsigned accumulate,
                                                hipStream_t stream);

/* Bytes of device workspace maglev_decode_step needs (0 on invalid sizes). */
size_t maglev_decode_workspace(int32_t Bs, int32_t H, int32_t Dh, int32_t W);

/* One recurrent decode step of one layer ([R-step] recurrent inference,
 * [R-mot] W-entry window, [G-inf] memory carried in the ordinary K/V cache).
 * Stream b is at absolute position p = pos[b] (read on the device, not
 * advanced). The new entry
 *   k~ = R_p k + s_h R_p kmem,  v~ = v + s_h vmem   (kmem/vmem: maglev_mem_project
 *   of m_{t-1} with shift = 0, T = 1)
 * is written to ring slot p mod W; then R_p q attends over the valid slots
 * (slot s holds position p - ((p - s) mod W), valid iff that is >= 0).
 *   q, k, v [Bs,H,Dh] dtype; gate_logit [H] float32;
 *   kmem, vmem: dtype, stream b's [H,Dh] block starts at element b * mem_stride
 *     (mem_stride >= H*Dh, a multiple of 8; 0 selects H*Dh, the packed layout).
 *     A stride above H*Dh lets one projection of m_{t-1} by every layer's
 *     stacked weights feed all layers of a step;
 *   kcache, vcache [Bs,H,W,Dh] dtype, read and updated in place;
 *   pos [Bs] int64 device; o [Bs,H,Dh] dtype, written.
 * workspace: device buffer of at least maglev_decode_workspace() bytes, owned
 *   by the caller (per-chunk partial softmax states; scratch on return; calls
 *   that overlap in time need their own workspaces).
 * The ring holds dtype values: the new entry is rounded once (ties to even).
 * The RoPE angle of the new position is evaluated on the device in double
 * precision, so no table bounds the position. A stream whose pos[b] is
 * negative is skipped: its ring slots and its row of o are left untouched.
 * Bs*H must be below 2^31 (one workgroup per stream and head), else
 * MAGLEV_ERR_INVALID_VALUE. */
maglev_status_t maglev_decode_step(int32_t Bs, int32_t H, int32_t Dh, int32_t W,
                                   float rope_base, float scale, int32_t dtype, const void *q,
                                   const void *k, const void *v, const void *kmem,
                                   const void *vmem, int64_t mem_stride,
                                   const float *gate_logit, void *kcache, void *vcache,
                                   const int64_t *pos, void *o, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Gated mixing form ([R-step]: the recurrent key is RMSNorm(W_k^rec m'_{t-1}),
 * the recurrent value W_v^rec m'_{t-1}; each layer mixes them with the local
 * features through channel-wise gates g = 2 sigmoid(a), neutral value 1 at
 * a = 0; [R-bg]: both keys are rotated before the mix):
 *   kp_j  = W_Km m'_{j-1},  vmem_j = W_Vm m'_{j-1}          (m'_{-1} := 0)
 *   kn_j  = kp_j / sqrt(mean_c kp_j[c]^2 + eps)             (over all H*Dh channels)
 *   k~_j  = g_kl (.) R_j k_j + g_kr (.) R_j kn_j,   v~_j = g_vl (.) v_j + g_vr (.) vmem_j
 * gates: float32 [4][H*Dh] logits in the order a_kl, a_kr, a_vl, a_vr; channel
 * c = h*Dh + i of a row. The norm has no learned scale (the recurrent gate
 * follows it). eps >= 0, finite. The gated calls need H*Dh <= 4096.
 * Attention over the gated entries is maglev_swa_inject_fwd, unchanged.
 * ------------------------------------------------------------------------- */

/* Projection with the shift (as maglev_mem_project) and the gated mix.
 *   m [B,T,d], W_Km, W_Vm [H*Dh,d], k, v [B,T,H,Dh]: dtype, read;
 *   kproj, vmem [B,T,H,Dh] dtype, written: the projections before the norm
 *     (the backward reads them);
 *   kmix, vmix [B,T,H,Dh] dtype, written: the gated entries above.
 * Every pointer is required (16-byte aligned) except for B*T == 0. */
maglev_status_t maglev_mem_project_gated(const maglev_geom_t *g, int shift, const void *m,
                                         const void *W_Km, const void *W_Vm, const void *k,
                                         const void *v, const float *gates, float eps,
                                         void *kproj, void *vmem, void *kmix, void *vmix,
                                         hipStream_t stream);

/* Bytes of device workspace maglev_swa_inject_bwd_gated needs (0 on invalid
 * geometry or H*Dh > 4096). It holds, besides the attention scratch, the
 * gradients of the two projections (2 * B*T*H*Dh dtype elements) and
 * per-workgroup gate partial sums. */
size_t maglev_swa_inject_bwd_gated_workspace(const maglev_geom_t *g);

/* Backward of the gated layer path: attention, gated mix, norm, shift and
 * projection (the chain rule through the forward above).
 * Inputs: q; kmix, vmix, kproj, vmem from maglev_mem_project_gated (shift 1);
 *   the local k, v; gates, eps; the forward's o and lse; dO; m_prime (unshifted);
 *   W_Km, W_Vm.
 * Outputs: dq, dk, dv [B,T,H,Dh] dtype (overwritten); dm_prime [B,T,d] float32
 *   (row T-1 gets no injection gradient); dW_Km, dW_Vm [H*Dh,d] float32;
 *   dgates [4][H*Dh] float32, the gradients of the four logit vectors.
 * accumulate: bit 0 dm_prime +=, bit 1 dW +=, bit 2 dgates +=.
 * workspace: at least maglev_swa_inject_bwd_gated_workspace(g) bytes.
 * Deterministic: partial sums are combined in a fixed order, no atomics. */
maglev_status_t maglev_swa_inject_bwd_gated(
    const maglev_geom_t *g, const void *q, const void *kmix, const void *vmix, const void *k,
    const void *v, const void *kproj, const void *vmem, const float *gates, float eps,
    const void *o, const float *lse, const void *dO, const void *m_prime, const void *W_Km,
    const void *W_Vm, void *dq, void *dk, void *dv, float *dm_prime, float *dW_Km, float *dW_Vm,
    float *dgates, unsigned accumulate, void *workspace, size_t workspace_bytes,
    hipStream_t stream);

/* One decode step of the gated form: as maglev_decode_step, with the new entry
 *   k~ = g_kl R_p k + g_kr R_p RMSNorm(kproj),  v~ = g_vl v + g_vr vmem,
 * where kproj, vmem are W_Km m_{t-1}, W_Vm m_{t-1} before the norm
 * (maglev_mem_project with shift = 0), stream b's H*Dh row starting at element
 * b * mem_stride (0 selects H*Dh), and the norm runs over that whole row.
 * gates [4][H*Dh] float32 logits; eps >= 0. Workspace as maglev_decode_step. */
maglev_status_t maglev_decode_step_gated(int32_t Bs, int32_t H, int32_t Dh, int32_t W,
                                         float rope_base, float scale, int32_t dtype,
                                         const void *q, const void *k, const void *v,
                                         const void *kproj, const void *vmem, int64_t mem_stride,
                                         const float *gates, float eps, void *kcache,
                                         void *vcache, const int64_t *pos, void *o,
                                         void *workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Layers sharing one memory projection ([R-step]: a shared projection maps
 * the shifted memory to the recurrent K/V features, each layer mixes them in
 * through its own gate). Per pass:
 *   maglev_mem_project(shift = 1, no mixing arguments) once -> kmem, vmem;
 *   per layer l: maglev_mix_entries(k_l, v_l, kmem, vmem, gate_l) and
 *     maglev_swa_inject_fwd; backward maglev_swa_inject_bwd_shared, which
 *     sums s dk and s dv of every layer into float32 dkmem, dvmem;
 *   maglev_mem_project_bwd once: dm' and dW from the sums.
 * The stack's objective is the sum over layers, so these are its gradients.
 * ------------------------------------------------------------------------- */

/* The mix of one layer from given memory terms (the mixing half of
 * maglev_mem_project): kmix = R_{pos0+t} k + s_h R_{pos0+t} kmem,
 * vmix = v + s_h vmem. k, v, kmem, vmem, kmix, vmix [B,T,H,Dh] dtype;
 * gate_logit [H] float32. Uses g->B, T, H, Dh, pos0, rope_base, dtype. */
maglev_status_t maglev_mix_entries(const maglev_geom_t *g, const void *k, const void *v,
                                   const void *kmem, const void *vmem, const float *gate_logit,
                                   void *kmix, void *vmix, hipStream_t stream);

/* Bytes of device workspace maglev_swa_inject_bwd_shared needs (0 on invalid geometry). */
size_t maglev_swa_inject_bwd_shared_workspace(const maglev_geom_t *g);

/* Backward of one layer whose memory terms come from a shared projection:
 *   dq, dk, dv [B,T,H,Dh] dtype (overwritten): gradients w.r.t. q, k, v;
 *   dkmem, dvmem [B,T,H,Dh] float32: s_h dk and s_h dv, the layer's share of
 *     the gradients of the shared kmem, vmem (accumulate bit 0: added);
 *   dgate [H] float32 (bit 2: added).
 * Inputs as maglev_swa_inject_bwd (kmix, vmix from maglev_mix_entries).
 * accumulate: only bits 0 and 2. Deterministic (fixed-order sums). */
maglev_status_t maglev_swa_inject_bwd_shared(const maglev_geom_t *g, const void *q,
                                             const void *kmix, const void *vmix,
                                             const void *kmem, const void *vmem,
                                             const float *gate_logit, const void *o,
                                             const float *lse, const void *dO, void *dq,
                                             void *dk, void *dv, float *dkmem, float *dvmem,
                                             float *dgate, unsigned accumulate, void *workspace,
                                             size_t workspace_bytes, hipStream_t stream);

/* The gated form over one shared projection ([R-step]: one projection of the
 * shifted memory for every layer, a per-layer gate, RMSNorm on the recurrent
 * key). Per pass:
 *   maglev_mem_project(shift = 1, no mixing arguments) once -> kproj, vmem
 *     (the projections before the norm);
 *   per layer l: maglev_mix_entries_gated(k_l, v_l, kproj, vmem, gates_l) and
 *     maglev_swa_inject_fwd; backward maglev_swa_inject_bwd_shared_gated,
 *     which sums every layer's gradients of kproj and vmem into float32
 *     dkproj, dvmem;
 *   maglev_mem_project_bwd(dkproj, dvmem) once: dm' and dW from the sums.
 * The norm is per layer's use of kproj (each layer normalises the same rows),
 * so its backward runs per layer and the sums are of pre-norm gradients. */

/* The gated mix of one layer from the shared pre-norm projections (the mixing
 * half of maglev_mem_project_gated): k, v, kproj, vmem, kmix, vmix
 * [B,T,H,Dh] dtype; gates [4][H*Dh] float32 logits; eps >= 0. H*Dh <= 4096. */
maglev_status_t maglev_mix_entries_gated(const maglev_geom_t *g, const void *k, const void *v,
                                         const void *kproj, const void *vmem, const float *gates,
                                         float eps, void *kmix, void *vmix, hipStream_t stream);

/* Bytes of device workspace maglev_swa_inject_bwd_shared_gated needs (0 on
 * invalid geometry or H*Dh > 4096). */
size_t maglev_swa_inject_bwd_shared_gated_workspace(const maglev_geom_t *g);

/* Backward of one gated layer whose recurrent terms come from a shared
 * projection (attention, gates, rotation and norm; no projection):
 *   dq, dk, dv [B,T,H,Dh] dtype (overwritten): gradients w.r.t. q, k, v;
 *   dkproj, dvmem [B,T,H,Dh] float32: the layer's share of the gradients of
 *     the shared kproj (before the norm) and vmem (accumulate bit 0: added);
 *   dgates [4][H*Dh] float32, the layer's gate-logit gradients (bit 2: added).
 * Inputs as maglev_swa_inject_bwd_gated without m_prime and the weights (kmix,
 * vmix from maglev_mix_entries_gated). accumulate: only bits 0 and 2.
 * Deterministic (fixed-order sums, no atomics). */
maglev_status_t maglev_swa_inject_bwd_shared_gated(
    const maglev_geom_t *g, const void *q, const void *kmix, const void *vmix, const void *k,
    const void *v, const void *kproj, const void *vmem, const float *gates, float eps,
    const void *o, const float *lse, const void *dO, void *dq, void *dk, void *dv, float *dkproj,
    float *dvmem, float *dgates, unsigned accumulate, void *workspace, size_t workspace_bytes,
    hipStream_t stream);

/* Bytes of device workspace maglev_mem_project_bwd needs (0 on invalid geometry). */
size_t maglev_mem_project_bwd_workspace(const maglev_geom_t *g);

/* Backward of the shift and projection from the gradients of the projected
 * memory: dkmem, dvmem [B,T,H,Dh] float32 (e.g. summed over the layers of a
 * pass); m_prime [B,T,d] dtype (unshifted); W_Km, W_Vm [H*Dh,d] dtype.
 *   dm_prime [B,T,d] float32: row t receives the gradient of projection
 *     input row t+1, row T-1 nothing (accumulate bit 0: added);
 *   dW_Km, dW_Vm [H*Dh,d] float32 (bit 1: added).
 * The bf16 path rounds dkmem, dvmem to bf16 once (MFMA operands). */
maglev_status_t maglev_mem_project_bwd(const maglev_geom_t *g, const float *dkmem,
                                       const float *dvmem, const void *m_prime, const void *W_Km,
                                       const void *W_Vm, float *dm_prime, float *dW_Km,
                                       float *dW_Vm, unsigned accumulate, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Attention without injection: the layers of the causal prefiller Q, which
 * produces the targets m' with interleaved sliding-window and full-attention
 * layers and no memory term ([R-core], [R-step]: the SLSL pattern, window 512
 * and full attention over the 2048 training context). A layer is
 *   O_i = sum_{j = max(0, i-W+1)}^{i} softmax_j(scale <R_i q_i, R_j k_j>) v_j,
 * a sliding-window layer with W = 512 and a full-attention layer with W >= T.
 * Forward: krot = maglev_rope_keys(k), then maglev_swa_inject_fwd(q, krot, v)
 * (the rotated keys and the plain values are the entries attended over).
 * ------------------------------------------------------------------------- */

/* krot = R_{pos0+t} k, [B,T,H,Dh] dtype (written; must not alias k).
 * Uses g->B, T, H, Dh, pos0, rope_base, dtype. */
maglev_status_t maglev_rope_keys(const maglev_geom_t *g, const void *k, void *krot,
                                 hipStream_t stream);

/* Bytes of device workspace maglev_attn_bwd needs (0 on invalid geometry). */
size_t maglev_attn_bwd_workspace(const maglev_geom_t *g);

/* Backward of attention without injection: from q, krot (maglev_rope_keys),
 * v, the forward's o and lse, and dO, writes dq, dk (w.r.t. the unrotated k)
 * and dv, all [B,T,H,Dh] dtype (overwritten). workspace: at least
 * maglev_attn_bwd_workspace(g) bytes. g->d is not used (any valid value). */
maglev_status_t maglev_attn_bwd(const maglev_geom_t *g, const void *q, const void *krot,
                                const void *v, const void *o, const float *lse, const void *dO,
                                void *dq, void *dk, void *dv, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace maglev_lm_head needs (0 on invalid sizes). The
 * float32 logits [N, V] dominate: 4 N V bytes, plus the dz buffer (N V
 * elements of dtype) and O(N d) more. */
size_t maglev_lm_head_workspace(int64_t N, int32_t d, int64_t V, int32_t dtype);

/* Loss head of the lifted pass ([R-step]: the output state m_t feeds the
 * soft-capped LM head, and the loss averages the cross-entropy and the
 * consistency term over the positions; [R-bg]: the targets m' are states
 * after the final RMSNorm):
 *   m_n    = h_n / sqrt(mean_e h_ne^2 + eps)        (RMSNorm, no learned scale)
 *   c_nv   = cap tanh((U m_n)_v / cap)
 *   CE_n   = logsumexp_v c_nv - c_n,target_n  (0 when target_n is outside [0, V))
 *   loss   = sum_n CE_n / N + lambda / (N sqrt(d)) sum_n ||m_n - m'_n||^2
 * Inputs: h [N, d] dtype (the decoder's last hidden state, one row per
 *   position); U [V, d] dtype (the head's weight, one row per vocabulary
 *   entry); targets [N] int64 (device); m_prime [N, d] dtype or NULL (then
 *   the consistency term is left out and lambda is unused).
 * Outputs: m [N, d] dtype = RMSNorm(h) (overwritten); loss: device float32
 *   scalar; dh [N, d] float32 and dU [V, d] float32, each optional (NULL:
 *   not computed; with both NULL no backward work is done): the gradients of
 *   loss w.r.t. h and U.
 * accumulate: bit 0 -> dh +=, bit 1 -> dU +=, bit 2 -> loss +=; a clear bit
 *   overwrites. Every position counts in N, also one whose target is ignored.
 * Constraints: N >= 1 (the mean over no positions is undefined), d a multiple
 *   of 16, V a multiple of 8 and >= 16, 0 < cap <= 64 (the log-sum-exp is
 *   taken without a running maximum, which needs exp(cap) V finite in
 *   float32), eps >= 0 and finite, lambda not NaN.
 * workspace: at least maglev_lm_head_workspace(N, d, V, dtype) bytes, owned by
 *   the caller, 16-byte aligned; contents are scratch on return. No
 *   floating-point atomics: the result is deterministic. */
maglev_status_t maglev_lm_head(int64_t N, int32_t d, int64_t V, float cap, float eps,
                               float lambda, int32_t dtype, const void *h, const void *U,
                               const int64_t *targets, const void *m_prime, void *m, float *loss,
                               float *dh, float *dU, unsigned accumulate, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* pos[b] += 1 for b < Bs on the device (moves every stream to its next ring
 * slot; kept separate so one decode step can be captured and replayed). */
maglev_status_t maglev_decode_advance(int32_t Bs, int64_t *pos, hipStream_t stream);

/* Set-up of the current device: ensure the RoPE table for (Dh, rope_base)
 * covers positions [0, max_pos), and look up the device scratch of
 * maglev_consistency_loss_noalloc. Synchronous; call before HIP-graph capture. */
maglev_status_t maglev_prepare(int32_t Dh, float rope_base, int64_t max_pos);

/* Human-readable name of a status code (static storage). */
const char *maglev_status_string(maglev_status_t status);

/* Text of the last HIP error seen by this thread (static per thread). */
const char *maglev_last_error(void);

/* MAGLEV_ABI_VERSION of the built library. */
int maglev_abi_version(void);

/* Kernel timing (diagnostic, for measurement tools). While switched on, every
 * kernel the library launches is timed with two HIP events on its launch
 * stream: the attention kernels and the GEMMs carry both events with their
 * dispatch (its own start and end times), the other kernels get one event
 * recorded on each side; launches on a stream under graph capture are not
 * recorded.
 *   maglev_profile_enable(1, only) clears earlier totals and starts recording
 *   every kernel (only == NULL) or just the kernel named `only` (host string,
 *   copied; fewer events leave fewer gaps in the stream);
 *   maglev_profile_enable(0, NULL) stops recording (totals are kept);
 *   maglev_profile_count() waits for the recorded events, folds them into
 *   per-kernel totals and returns the number of kernel names;
 *   maglev_profile_entry(i, ...) gives name i (static until the next enable),
 *   its launch count and its summed duration in milliseconds.
 * Recorded events add a small gap between kernels; timing is off by default. */
maglev_status_t maglev_profile_enable(int on, const char *only);
int maglev_profile_count(void);

/* Debug mode (diagnostic; off by default, on at load when the environment
 * variable MAGLEV_DEBUG is set to anything but "0"): after each kernel launch
 * (or the few launches of one step) the library takes the launch error and
 * synchronises the launch stream, so that a failure is reported by the call
 * that launched the faulting kernel, as MAGLEV_ERR_HIP with
 * maglev_last_error() = "<kernel name>: <HIP error>". Launches on a stream
 * under graph capture are not checked. Slow: every launch waits for the GPU.
 * maglev_debug_enable(on) switches it for the whole process;
 * maglev_debug_enabled() returns 1 while it is on. */
maglev_status_t maglev_debug_enable(int on);
int maglev_debug_enabled(void);

maglev_status_t maglev_profile_entry(int index, const char **name, int64_t *launches,
                                     double *total_ms);

#ifdef __cplusplus
}
#endif

#endif /* MAGLEV_H */
