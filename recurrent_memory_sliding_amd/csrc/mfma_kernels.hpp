// mfma_kernels.hpp -- launchers of the bf16 MFMA kernels (gfx950,
// v_mfma_f32_32x32x16_bf16, fp32 accumulation).
#pragma once

#include "internal.hpp"

namespace maglev {
namespace mfma {

// kmem/vmem = input * [W_Km; W_Vm]^T with the shift folded into the row loads.
void launch_project_bf16(const Geom &g, int shift, const void *m, const void *wk, const void *wv,
                         void *km, void *vm, hipStream_t s);

// Banded flash-style forward over the mixed entries (K/V tiles staged by
// direct global->LDS loads, double-buffered).
void launch_attn_fwd_bf16(const Geom &g, const void *q, const void *kx, const void *vx,
                          const float2 *rope, void *o, float *lse, hipStream_t s);

// Attention backward: rotated queries and rowsum(dO*O), key-stationary dK/dV
// pass, query-stationary dQ pass. entries = true: dk/dv receive the gradients
// of the mixed entries (rotated frame) instead of those of k and v.
void launch_attn_bwd_bf16(const Geom &g, const void *q, const void *kx, const void *vx,
                          const void *o, const float *lse, const void *dO, void *dq, void *dk,
                          void *dv, const BwdWorkspace &ws, const float2 *rope, bool entries,
                          hipStream_t s);

// Projection backward: dm' (shifted back) and dW_Km/dW_Vm (split-K, fixed-order
// reduction). With a gate it also writes ws.rowdot[r] = <W[r,:], G[r,:]>, the
// row's share of the gate gradient (G = sum_t [dk|dv]_t x_t^T before the sigma
// factor). gate == nullptr: dk/dv are the gradients of the projected memory
// itself (no per-head sigma factor, no row dots).
void launch_proj_bwd_bf16(const Geom &g, const void *dk, const void *dv, const void *m_prime,
                          const void *wk, const void *wv, const float *gate, float *dm_prime,
                          float *dWk, float *dWv, unsigned acc, const BwdWorkspace &ws,
                          hipStream_t s);

// Loss-head products: logits = cap tanh(m U^T / cap) (float32 [N,V]) with
// rowsum[n, t] = sum of exp(logit) over column tile t of row n (float32
// [N, lm_logits_col_tiles(V)], cap <= 64), dm = dz U (float32 [N,d]),
// dU (+)= dz^T m (float32 [V,d]). ut: [d][V] bf16 scratch that the dm product
// fills with U transposed when it takes its large tiles.
int64_t lm_logits_col_tiles(int64_t V);
void launch_lm_logits_bf16(int64_t N, int64_t V, int d, float cap, const void *m, const void *u,
                           float *logits, float *rowsum, hipStream_t s);
void launch_lm_dm_bf16(int64_t N, int64_t V, int d, const void *dz, const void *u, void *ut,
                       float *dm, hipStream_t s);
void launch_lm_du_bf16(int64_t N, int64_t V, int d, const void *dz, const void *m, float *du,
                       bool acc, hipStream_t s);

// Widest window (in 32-query tiles per 32-key tile) whose dS tiles the dK/dV
// pass stores for the dQ pass (Dh = 128); wider windows recompute the scores.
constexpr int kMaxDsTiles = 80;

// Split-K factor the dW GEMM uses for this geometry (workspace sizing).
int dw_ksplit(const Geom &g);

}  // namespace mfma
}  // namespace maglev
