// path.hip -- launchers of the training-pass kernels: memory projection,
// attention forward and the backward sequence. bf16 runs on the MFMA kernels
// (mfma_*.hip); float32 runs on the vector-ALU kernels of simt_kernels.hpp.
//
// Method: Maglev summary on paper.rainbus.top ("Maglev：滑动窗口循环记忆"),
// section 方法步骤详情 (P consumes the shifted targets m'_{0:T-1}, m'_0 = 0;
// projection W^rec m'_{t-1} into K/V features; gated mix; sliding-window
// attention over the W most recent mixed entries) and gist.science
// ("Technische Samenvatting: Maglev - Sliding Recurrent Memory"), section
// Trainingsmechanisme (the second parallel pass through P). The backward is
// the chain rule through those steps.
#include "common.hpp"
#include "internal.hpp"
#include "mfma_kernels.hpp"
#include "profile.hpp"
#include "simt_kernels.hpp"

namespace maglev {

namespace {

template <typename T>
struct ProjA {  // row (b,t) of the projection input: m[b, t - shift] or 0
    const T *m;
    int64_t T_;
    int d, shift;
    __device__ float operator()(int64_t row, int64_t e) const
    {
        const int64_t t = row % T_;
        return t >= shift ? to_f<T>(m[(row - shift) * d + e]) : 0.0f;
    }
};
template <typename T>
struct ProjB {  // column n of the stacked weight [W_Km; W_Vm]^T
    const T *wk, *wv;
    int HD, d;
    __device__ float operator()(int64_t e, int64_t n) const
    {
        return n < HD ? to_f<T>(wk[n * d + e]) : to_f<T>(wv[(n - HD) * d + e]);
    }
};
template <typename T>
struct ProjStore {
    T *km, *vm;
    int HD;
    __device__ void operator()(int64_t row, int64_t n, float x) const
    {
        if (n < HD) km[row * HD + n] = from_f<T>(x);
        else vm[row * HD + (n - HD)] = from_f<T>(x);
    }
};

// d loss / d input row (b,t) = sum_r s_h(r) (dk[b,t,r] W_Km[r,:] + dv[b,t,r] W_Vm[r,:]);
// it lands on dm'[b, t-1] (t >= 1).
template <typename T>
struct DmA {
    const T *dk, *dv;
    int HD;
    __device__ float operator()(int64_t row, int64_t r) const
    {
        return r < HD ? to_f<T>(dk[row * HD + r]) : to_f<T>(dv[row * HD + r - HD]);
    }
};
template <typename T>
struct DmB {
    const T *wk, *wv;
    const float *gate;
    int HD, Dh, d;
    __device__ float operator()(int64_t r, int64_t e) const
    {
        const int rr = (int)(r < HD ? r : r - HD);
        const float s = gate ? gate_sigmoid(gate[rr / Dh]) : 1.0f;
        return s * (r < HD ? to_f<T>(wk[r * d + e]) : to_f<T>(wv[rr * (int64_t)d + e]));
    }
};
struct DmStore {
    float *dm;
    int64_t T_;
    int d;
    bool acc;
    __device__ void operator()(int64_t row, int64_t e, float x) const
    {
        if (row % T_ == 0) return;   // d/d input row (b,0) has no source memory
        float *p = dm + (row - 1) * d + e;
        *p = acc ? *p + x : x;
    }
};

// dW[r, e] = s_h(r) sum_{b,t} dkv[b,t,r] input[b,t,e].
template <typename T>
struct DwA {
    const T *dk, *dv;
    int HD;
    __device__ float operator()(int64_t r, int64_t row) const
    {
        return r < HD ? to_f<T>(dk[row * HD + r]) : to_f<T>(dv[row * HD + r - HD]);
    }
};
struct DwStore {
    float *wk, *wv;
    const float *gate;
    int HD, Dh, d;
    bool acc;
    __device__ void operator()(int64_t r, int64_t e, float x) const
    {
        const int rr = (int)(r < HD ? r : r - HD);
        if (gate) x *= gate_sigmoid(gate[rr / Dh]);
        float *p = (r < HD ? wk : wv) + (int64_t)rr * d + e;
        *p = acc ? *p + x : x;
    }
};

__global__ void fill_zero(float *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

__global__ void zero_last_rows(float *dm, int64_t B, int64_t T, int d)
{
    const int64_t b = blockIdx.x;
    for (int e = threadIdx.x; e < d; e += blockDim.x) dm[(b * T + T - 1) * d + e] = 0.0f;
}

// dgate[h] = s(1-s) * sum of the per-row or per-tile partials of head h, in a
// fixed order (deterministic).
__global__ __launch_bounds__(256) void dgate_reduce(const float *part, int64_t B, int H,
                                                    int64_t per_bh, const float *gate,
                                                    float *dgate, unsigned acc)
{
    __shared__ float red[4];
    const int h = blockIdx.x;
    float t = 0.0f;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = threadIdx.x; i < per_bh; i += 256) t += part[(b * H + h) * per_bh + i];
    t = wave_sum(t);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float s = gate_sigmoid(gate[h]);
        const float g = s * (1.0f - s) * (red[0] + red[1] + red[2] + red[3]);
        dgate[h] = (acc & 4u) ? dgate[h] + g : g;
    }
}

// dgate[h] = s(1-s) * sum over the rows r of head h of rowdot[r] + rowdot[HD + r]
// (the key and the value weight rows), summed in a fixed order. One wave per head.
__global__ __launch_bounds__(64) void dgate_from_rows(const float *rowdot, int HD, int Dh,
                                                      const float *gate, float *dgate,
                                                      unsigned acc)
{
    const int h = blockIdx.x, lane = threadIdx.x;
    float t = 0.0f;
    for (int i = lane; i < Dh; i += 64) t += rowdot[h * Dh + i] + rowdot[HD + h * Dh + i];
    t = wave_sum(t);
    if (lane == 0) {
        const float sg = gate_sigmoid(gate[h]);
        const float g = sg * (1.0f - sg) * t;
        dgate[h] = (acc & 4u) ? dgate[h] + g : g;
    }
}

// One layer's contribution to the gradients of a memory projection shared by
// several layers: dkm (+)= s_h dk, dvm (+)= s_h dv (float32 [B,T,H,Dh]), and
// part[(b H + h) nblk + tb] = sum over this block's tokens of
// <kmem, dk> + <vmem, dv> (the gate terms of head h). One workgroup per
// (token block, b, h); 16 bytes a lane.
template <typename T, int DH>
__global__ __launch_bounds__(256) void shared_mem_grad(int64_t Tlen, int H, int tokens,
                                                       const float *gate, const T *dk, const T *dv,
                                                       const T *km, const T *vm, float *dkm,
                                                       float *dvm, float *part, unsigned acc)
{
    constexpr int CPT = DH / 8;           // 8-channel chunks of one token's head row
    constexpr int TPP = 256 / CPT;        // tokens per pass
    __shared__ float red[4];
    const int bh = blockIdx.y, h = bh % H;
    const int64_t b = bh / H;
    const int c = threadIdx.x % CPT, tl = threadIdx.x / CPT;
    const float sg = gate_sigmoid(gate[h]);
    const int64_t t0 = (int64_t)blockIdx.x * tokens;
    const int64_t t1 = t0 + tokens < Tlen ? t0 + tokens : Tlen;
    float p = 0.0f;
    for (int64_t t = t0 + tl; t < t1; t += TPP) {
        const int64_t off = ((b * Tlen + t) * H + h) * DH + 8 * c;
        float x[8], y[8], z[8];
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            load8((pass ? dv : dk) + off, x);
            load8((pass ? vm : km) + off, y);
            float *dst = (pass ? dvm : dkm) + off;
            if (acc) load8(dst, z);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p += x[e] * y[e];
                z[e] = acc ? z[e] + sg * x[e] : sg * x[e];
            }
            store8(dst, z);
        }
    }
    p = wave_sum(p);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = p;
    __syncthreads();
    if (threadIdx.x == 0) part[(int64_t)bh * gridDim.x + blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// float32 -> bf16, 8 elements a thread (n a multiple of 8).
__global__ void to_bf16(const float *x, bf16 *y, int64_t n8)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    float v[8];
    load8(x + 8 * i, v);
    store8(y + 8 * i, v);
}

simt::RowArgs row_args(const Geom &g, const float *gate, const float2 *rope)
{
    simt::RowArgs a;
    a.B = g.B; a.T = g.T; a.H = g.H; a.W = g.W; a.pos0 = g.pos0; a.scale = g.scale;
    a.rope = rope; a.gate = gate;
    return a;
}

template <typename T>
void project_simt(const Geom &g, int shift, const void *m, const void *wk, const void *wv,
                  void *km, void *vm, hipStream_t s)
{
    const int64_t M = g.N(), N = 2 * g.HD(), K = g.d;
    ProjA<T> la{static_cast<const T *>(m), g.T, g.d, shift};
    ProjB<T> lb{static_cast<const T *>(wk), static_cast<const T *>(wv), g.HD(), g.d};
    ProjStore<T> st{static_cast<T *>(km), static_cast<T *>(vm), g.HD()};
    hipLaunchKernelGGL((simt::gemm_tiled<ProjA<T>, ProjB<T>, ProjStore<T>>),
                       dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, s, M, N, K, la, lb, st);
}

template <typename T, int DH>
void fwd_simt(const Geom &g, const void *q, const void *kx, const void *vx, const float2 *rope,
              void *o, float *lse, hipStream_t s)
{
    hipLaunchKernelGGL((simt::attn_fwd_rows<T, DH>), dim3(g.T, g.H, g.B), dim3(DH), 0, s,
                       row_args(g, nullptr, rope), static_cast<const T *>(q),
                       static_cast<const T *>(kx), static_cast<const T *>(vx),
                       static_cast<T *>(o), lse);
}

template <typename T, int DH>
void mix_launch(const Geom &g, const void *k, const void *v, const void *km, const void *vm,
                const float *gate, const float2 *rope, void *kx, void *vx, hipStream_t s)
{
    const int64_t rows = g.N() * g.H;
    const int64_t threads = rows * (DH / 16);
    prof::Scope ts("mix", s);
    hipLaunchKernelGGL((simt::mix_entries<T, DH>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, rows, g.H, g.T, g.pos0, rope, gate,
                       static_cast<const T *>(k), static_cast<const T *>(v),
                       static_cast<const T *>(km), static_cast<const T *>(vm),
                       static_cast<T *>(kx), static_cast<T *>(vx));
}

// ROTATE false: dk/dv receive the gradients of the mixed entries; PARTIAL:
// the per-key gate terms of the sigma form go to ws.ds_part (reads km, vm).
template <typename T, int DH, bool ROTATE = true, bool PARTIAL = true>
void attn_bwd_simt(const Geom &g, const void *q, const void *kx, const void *vx, const void *km,
                   const void *vm, const float *gate, const void *o, const float *lse,
                   const void *dO, void *dq, void *dk, void *dv, const BwdWorkspace &ws,
                   const float2 *rope, hipStream_t s)
{
    const simt::RowArgs a = row_args(g, gate, rope);
    const dim3 grid(g.T, g.H, g.B);
    hipLaunchKernelGGL((simt::bwd_rowdot<T, DH>), grid, dim3(DH), 0, s, a,
                       static_cast<const T *>(o), static_cast<const T *>(dO), ws.D);
    hipLaunchKernelGGL((simt::bwd_dq_rows<T, DH>), grid, dim3(DH), 0, s, a,
                       static_cast<const T *>(q), static_cast<const T *>(kx),
                       static_cast<const T *>(vx), static_cast<const T *>(dO), lse, ws.D,
                       static_cast<T *>(dq));
    hipLaunchKernelGGL((simt::bwd_dkdv_rows<T, DH, ROTATE, PARTIAL>), grid, dim3(DH), 0, s, a,
                       static_cast<const T *>(q), static_cast<const T *>(kx),
                       static_cast<const T *>(vx), static_cast<const T *>(km),
                       static_cast<const T *>(vm), static_cast<const T *>(dO), lse, ws.D,
                       static_cast<T *>(dk), static_cast<T *>(dv), ws.ds_part);
}

template <typename T>
void proj_bwd_simt(const Geom &g, const void *dk, const void *dv, const void *m_prime,
                   const void *wk, const void *wv, const float *gate, float *dm_prime,
                   float *dWk, float *dWv, unsigned acc, hipStream_t s)
{
    const int HD = g.HD();
    {
        const int64_t M = g.N(), N = g.d, K = 2 * HD;
        DmA<T> la{static_cast<const T *>(dk), static_cast<const T *>(dv), HD};
        DmB<T> lb{static_cast<const T *>(wk), static_cast<const T *>(wv), gate, HD, g.Dh, g.d};
        DmStore st{dm_prime, g.T, g.d, (acc & 1u) != 0};
        hipLaunchKernelGGL((simt::gemm_tiled<DmA<T>, DmB<T>, DmStore>),
                           dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, s, M, N, K, la, lb, st);
    }
    {
        const int64_t M = 2 * HD, N = g.d, K = g.N();
        DwA<T> la{static_cast<const T *>(dk), static_cast<const T *>(dv), HD};
        ProjA<T> lb{static_cast<const T *>(m_prime), g.T, g.d, 1};
        DwStore st{dWk, dWv, gate, HD, g.Dh, g.d, (acc & 2u) != 0};
        hipLaunchKernelGGL((simt::gemm_tiled<DwA<T>, ProjA<T>, DwStore>),
                           dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, s, M, N, K, la, lb, st);
    }
}

}  // namespace

hipError_t launch_project(const Geom &g, int shift, const void *m, const void *wk, const void *wv,
                          void *km, void *vm, hipStream_t s)
{
    if (g.dtype == MAGLEV_BF16)
        mfma::launch_project_bf16(g, shift, m, wk, wv, km, vm, s);
    else
        project_simt<float>(g, shift, m, wk, wv, km, vm, s);
    return hipGetLastError();
}

hipError_t launch_mix(const Geom &g, const void *k, const void *v, const void *km, const void *vm,
                      const float *gate, const float2 *rope, void *kx, void *vx, hipStream_t s)
{
    if (g.dtype == MAGLEV_BF16) {
        if (g.Dh == 128) mix_launch<bf16, 128>(g, k, v, km, vm, gate, rope, kx, vx, s);
        else mix_launch<bf16, 64>(g, k, v, km, vm, gate, rope, kx, vx, s);
    } else {
        if (g.Dh == 128) mix_launch<float, 128>(g, k, v, km, vm, gate, rope, kx, vx, s);
        else mix_launch<float, 64>(g, k, v, km, vm, gate, rope, kx, vx, s);
    }
    return hipGetLastError();
}

hipError_t launch_attn_fwd(const Geom &g, const void *q, const void *kx, const void *vx,
                           const float2 *rope, void *o, float *lse, hipStream_t s)
{
    if (g.dtype == MAGLEV_BF16) {
        mfma::launch_attn_fwd_bf16(g, q, kx, vx, rope, o, lse, s);
    } else {
        if (g.Dh == 128) fwd_simt<float, 128>(g, q, kx, vx, rope, o, lse, s);
        else fwd_simt<float, 64>(g, q, kx, vx, rope, o, lse, s);
    }
    return hipGetLastError();
}

size_t bwd_workspace_bytes(const Geom &g, BwdWorkspace *L, char *base, BwdKind kind)
{
    auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
    const bool bf = g.dtype == MAGLEV_BF16;
    // a projection backward follows (sigma, gated) or is the whole call (proj)
    const bool proj = kind == BwdKind::Sigma || kind == BwdKind::Gated || kind == BwdKind::Proj;
    const bool attn = kind != BwdKind::Proj;          // an attention backward runs
    const bool gated = kind == BwdKind::Gated;
    // the gated mix backward runs (its gate partials are needed)
    const bool gmix = gated || kind == BwdKind::SharedGated;
    const bool shared = kind == BwdKind::Shared;
    const size_t esz = bf ? 2 : 4;
    const size_t BHT = (size_t)g.B * g.H * g.T;
    const size_t HD = (size_t)g.HD();
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align(off + bytes); return o; };
    auto at = [&](size_t o, bool used) { return base && used ? base + o : nullptr; };
    L->n_key_tiles = (int)((g.T + 127) / 128);
    L->ksplit = bf && proj ? mfma::dw_ksplit(g) : 0;
    L->Tp = (g.T + 31) / 32 * 32;
    L->g_rows = L->g_blocks = 0;
    if (gmix) gated_partition(g.N(), &L->g_rows, &L->g_blocks);
    // float32 path: row sums D and, for the sigma form, the per-key gate terms;
    // a layer of a shared projection: per-block gate terms (both paths)
    const size_t nsp = (size_t)g.B * g.H * ((g.T + kSharedTokens - 1) / kSharedTokens);
    const size_t oD = take(!bf && attn ? BHT * sizeof(float) : 0);
    const size_t oS = take(!bf && kind == BwdKind::Sigma ? BHT * sizeof(float)
                           : shared ? nsp * sizeof(float) : 0);
    // bf16 path: rotated queries, padded lse*log2(e) and D
    const size_t nq = bf && attn ? (size_t)g.N() * HD : 0;
    const size_t npad = bf && attn ? (size_t)g.B * g.H * L->Tp : 0;
    const size_t oQ = take(nq * esz);
    const size_t oL = take(npad * sizeof(float));
    const size_t oDp = take(npad * sizeof(float));
    // bf16 path, Dh = 128: the dS tiles the dQ pass reads (windows up to
    // kMaxDsTiles query tiles a key tile; wider ones make the dQ pass
    // recompute the scores instead)
    L->nt32 = (int)((g.T + 31) / 32);
    L->ds_tiles = (g.W + 30) / 32 + 1 < L->nt32 ? (g.W + 30) / 32 + 1 : L->nt32;
    const bool ds = bf && attn && g.Dh == 128 && L->ds_tiles <= mfma::kMaxDsTiles;
    const size_t oDS = take(ds ? (size_t)g.B * g.H * L->nt32 * L->ds_tiles * 1024 * esz : 0);
    // projection backward (bf16): scaled weight copy, split-K partials, row dots
    const size_t oW = take(bf && proj ? 2 * HD * g.d * esz : 0);
    const size_t oP = take((size_t)L->ksplit * 2 * HD * g.d * sizeof(float));
    const size_t oR = take(bf && kind == BwdKind::Sigma ? 2 * HD * sizeof(float) : 0);
    // gated form: gradients of the two projections and the gate partials; the
    // shared projection's backward (bf16): its float32 gradients rounded to bf16
    const size_t nact = gated || (bf && kind == BwdKind::Proj) ? (size_t)g.N() * HD : 0;
    const size_t oKp = take(nact * esz);
    const size_t oVm = take(nact * esz);
    const size_t oG = take((size_t)L->g_blocks * 4 * HD * sizeof(float));
    L->D = reinterpret_cast<float *>(at(oD, !bf && attn));
    L->ds_part = reinterpret_cast<float *>(at(oS, (!bf && kind == BwdKind::Sigma) || shared));
    L->q_rot = at(oQ, nq > 0);
    L->ds = at(oDS, ds);
    L->lse2 = reinterpret_cast<float *>(at(oL, npad > 0));
    L->Dp = reinterpret_cast<float *>(at(oDp, npad > 0));
    L->W_scaled = at(oW, bf && proj);
    L->dW_part = reinterpret_cast<float *>(at(oP, L->ksplit > 0));
    L->rowdot = reinterpret_cast<float *>(at(oR, bf && kind == BwdKind::Sigma));
    L->dkp = at(oKp, nact > 0);
    L->dvm = at(oVm, nact > 0);
    L->gpart = reinterpret_cast<float *>(at(oG, gmix));
    return off;
}

hipError_t launch_bwd(const Geom &g, const void *q, const void *kx, const void *vx, const void *km,
                      const void *vm, const float *gate, const void *o, const float *lse,
                      const void *dO, const void *m_prime, const void *wk, const void *wv,
                      void *dq, void *dk, void *dv, float *dm_prime, float *dWk, float *dWv,
                      float *dgate, unsigned acc, const BwdWorkspace &ws, const float2 *rope,
                      hipStream_t s)
{
    const int HD = g.HD();
    if (g.N() == 0) {
        // No tokens: the parameter gradients are zero (left alone when accumulating).
        const int64_t nw = (int64_t)HD * g.d;
        if (!(acc & 2u)) {
            hipLaunchKernelGGL(fill_zero, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, dWk, nw);
            hipLaunchKernelGGL(fill_zero, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, dWv, nw);
        }
        if (!(acc & 4u)) hipLaunchKernelGGL(fill_zero, dim3(1), dim3(256), 0, s, dgate, (int64_t)g.H);
        return hipGetLastError();
    }
    if (g.dtype == MAGLEV_BF16) {
        // attention, then the projection backward, whose dW reduction also
        // gives each weight row's share <W[r,:], G[r,:]> of the gate gradient
        mfma::launch_attn_bwd_bf16(g, q, kx, vx, o, lse, dO, dq, dk, dv, ws, rope, false, s);
        mfma::launch_proj_bwd_bf16(g, dk, dv, m_prime, wk, wv, gate, dm_prime, dWk, dWv, acc, ws, s);
        prof::Scope ts("dgate_reduce", s);
        hipLaunchKernelGGL(dgate_from_rows, dim3(g.H), dim3(64), 0, s, ws.rowdot, HD, g.Dh, gate,
                           dgate, acc);
        return hipGetLastError();
    }
    if (g.Dh == 128)
        attn_bwd_simt<float, 128>(g, q, kx, vx, km, vm, gate, o, lse, dO, dq, dk, dv, ws, rope, s);
    else
        attn_bwd_simt<float, 64>(g, q, kx, vx, km, vm, gate, o, lse, dO, dq, dk, dv, ws, rope, s);
    {
        prof::Scope ts("dgate_reduce", s);
        hipLaunchKernelGGL(dgate_reduce, dim3(g.H), dim3(256), 0, s, ws.ds_part, g.B, g.H, g.T,
                           gate, dgate, acc);
    }
    if (!(acc & 1u)) {
        prof::Scope ts("zero_last_rows", s);
        hipLaunchKernelGGL(zero_last_rows, dim3(g.B), dim3(256), 0, s, dm_prime, g.B, g.T, g.d);
    }
    proj_bwd_simt<float>(g, dk, dv, m_prime, wk, wv, gate, dm_prime, dWk, dWv, acc, s);
    return hipGetLastError();
}

hipError_t launch_bwd_gated(const Geom &g, const void *q, const void *kx, const void *vx,
                            const void *k, const void *v, const void *kp, const void *vm,
                            const float *gates, float eps, const void *o, const float *lse,
                            const void *dO, const void *m_prime, const void *wk, const void *wv,
                            void *dq, void *dk, void *dv, float *dm_prime, float *dWk, float *dWv,
                            float *dgates, unsigned acc, const BwdWorkspace &ws,
                            const float2 *rope, hipStream_t s)
{
    const int HD = g.HD();
    if (g.N() == 0) {
        const int64_t nw = (int64_t)HD * g.d;
        if (!(acc & 2u)) {
            hipLaunchKernelGGL(fill_zero, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, dWk, nw);
            hipLaunchKernelGGL(fill_zero, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, dWv, nw);
        }
        if (!(acc & 4u))
            hipLaunchKernelGGL(fill_zero, dim3((unsigned)((4 * HD + 255) / 256)), dim3(256), 0, s,
                               dgates, (int64_t)4 * HD);
        return hipGetLastError();
    }
    // 1. attention backward: dq, and the gradients of the mixed entries into dk/dv
    if (g.dtype == MAGLEV_BF16) {
        mfma::launch_attn_bwd_bf16(g, q, kx, vx, o, lse, dO, dq, dk, dv, ws, rope, true, s);
    } else if (g.Dh == 128) {
        attn_bwd_simt<float, 128, false, false>(g, q, kx, vx, nullptr, nullptr, nullptr, o, lse, dO,
                                                dq, dk, dv, ws, rope, s);
    } else {
        attn_bwd_simt<float, 64, false, false>(g, q, kx, vx, nullptr, nullptr, nullptr, o, lse, dO,
                                               dq, dk, dv, ws, rope, s);
    }
    // 2. gates, rotation and norm backward: dk, dv final; gradients of the projection
    hipError_t e = launch_gated_mix_bwd(g, k, v, kp, vm, gates, eps, rope, dk, dv, ws, dgates, acc,
                                        nullptr, nullptr, s);
    if (e != hipSuccess) return e;
    // 3. shift and projection backward (no further gate factor)
    if (!(acc & 1u) && g.dtype != MAGLEV_BF16) {
        prof::Scope ts("zero_last_rows", s);
        hipLaunchKernelGGL(zero_last_rows, dim3(g.B), dim3(256), 0, s, dm_prime, g.B, g.T, g.d);
    }
    if (g.dtype == MAGLEV_BF16)
        mfma::launch_proj_bwd_bf16(g, ws.dkp, ws.dvm, m_prime, wk, wv, nullptr, dm_prime, dWk, dWv,
                                   acc, ws, s);
    else
        proj_bwd_simt<float>(g, ws.dkp, ws.dvm, m_prime, wk, wv, nullptr, dm_prime, dWk, dWv, acc, s);
    return hipGetLastError();
}

hipError_t launch_rope_keys(const Geom &g, const void *k, const float2 *rope, void *kr,
                            hipStream_t s)
{
    const int64_t rows = g.N() * g.H;
    const int64_t threads = rows * (g.Dh / 16);
    const dim3 grid((unsigned)((threads + 255) / 256));
    prof::Scope ts("rope_keys", s);
    if (g.dtype == MAGLEV_BF16) {
        if (g.Dh == 128)
            hipLaunchKernelGGL((simt::rope_rows<bf16, 128>), grid, dim3(256), 0, s, rows, g.H, g.T,
                               g.pos0, rope, static_cast<const bf16 *>(k), static_cast<bf16 *>(kr));
        else
            hipLaunchKernelGGL((simt::rope_rows<bf16, 64>), grid, dim3(256), 0, s, rows, g.H, g.T,
                               g.pos0, rope, static_cast<const bf16 *>(k), static_cast<bf16 *>(kr));
    } else {
        if (g.Dh == 128)
            hipLaunchKernelGGL((simt::rope_rows<float, 128>), grid, dim3(256), 0, s, rows, g.H, g.T,
                               g.pos0, rope, static_cast<const float *>(k), static_cast<float *>(kr));
        else
            hipLaunchKernelGGL((simt::rope_rows<float, 64>), grid, dim3(256), 0, s, rows, g.H, g.T,
                               g.pos0, rope, static_cast<const float *>(k), static_cast<float *>(kr));
    }
    return hipGetLastError();
}

hipError_t launch_attn_bwd(const Geom &g, const void *q, const void *kr, const void *v,
                           const void *o, const float *lse, const void *dO, void *dq, void *dk,
                           void *dv, const BwdWorkspace &ws, const float2 *rope, hipStream_t s)
{
    if (g.N() == 0) return hipSuccess;
    if (g.dtype == MAGLEV_BF16)
        mfma::launch_attn_bwd_bf16(g, q, kr, v, o, lse, dO, dq, dk, dv, ws, rope, false, s);
    else if (g.Dh == 128)
        attn_bwd_simt<float, 128, true, false>(g, q, kr, v, nullptr, nullptr, nullptr, o, lse, dO, dq,
                                               dk, dv, ws, rope, s);
    else
        attn_bwd_simt<float, 64, true, false>(g, q, kr, v, nullptr, nullptr, nullptr, o, lse, dO, dq,
                                              dk, dv, ws, rope, s);
    return hipGetLastError();
}

template <typename T, int DH>
static void shared_grad_t(const Geom &g, const float *gate, const void *dk, const void *dv,
                          const void *km, const void *vm, float *dkm, float *dvm, float *part,
                          unsigned acc, hipStream_t s)
{
    const dim3 grid((unsigned)((g.T + kSharedTokens - 1) / kSharedTokens), (unsigned)(g.B * g.H));
    prof::Scope ts("shared_mem_grad", s);
    hipLaunchKernelGGL((shared_mem_grad<T, DH>), grid, dim3(256), 0, s, g.T, g.H, kSharedTokens,
                       gate, static_cast<const T *>(dk), static_cast<const T *>(dv),
                       static_cast<const T *>(km), static_cast<const T *>(vm), dkm, dvm, part, acc);
}

hipError_t launch_bwd_shared(const Geom &g, const void *q, const void *kx, const void *vx,
                             const void *km, const void *vm, const float *gate, const void *o,
                             const float *lse, const void *dO, void *dq, void *dk, void *dv,
                             float *dkm, float *dvm, float *dgate, unsigned acc,
                             const BwdWorkspace &ws, const float2 *rope, hipStream_t s)
{
    if (g.N() == 0) {   // no tokens: only dgate is written (zero), unless it accumulates
        if (acc & 4u) return hipSuccess;
        hipLaunchKernelGGL(fill_zero, dim3(1), dim3(256), 0, s, dgate, (int64_t)g.H);
        return hipGetLastError();
    }
    hipError_t e = launch_attn_bwd(g, q, kx, vx, o, lse, dO, dq, dk, dv, ws, rope, s);
    if (e != hipSuccess) return e;
    const unsigned a1 = acc & 1u;
    if (g.dtype == MAGLEV_BF16) {
        if (g.Dh == 128) shared_grad_t<bf16, 128>(g, gate, dk, dv, km, vm, dkm, dvm, ws.ds_part, a1, s);
        else shared_grad_t<bf16, 64>(g, gate, dk, dv, km, vm, dkm, dvm, ws.ds_part, a1, s);
    } else {
        if (g.Dh == 128) shared_grad_t<float, 128>(g, gate, dk, dv, km, vm, dkm, dvm, ws.ds_part, a1, s);
        else shared_grad_t<float, 64>(g, gate, dk, dv, km, vm, dkm, dvm, ws.ds_part, a1, s);
    }
    prof::Scope ts("dgate_reduce", s);
    hipLaunchKernelGGL(dgate_reduce, dim3(g.H), dim3(256), 0, s, ws.ds_part, g.B, g.H,
                       (int64_t)((g.T + kSharedTokens - 1) / kSharedTokens), gate, dgate, acc);
    return hipGetLastError();
}

hipError_t launch_bwd_shared_gated(const Geom &g, const void *q, const void *kx, const void *vx,
                                   const void *k, const void *v, const void *kp, const void *vm,
                                   const float *gates, float eps, const void *o, const float *lse,
                                   const void *dO, void *dq, void *dk, void *dv, float *dkp,
                                   float *dvm, float *dgates, unsigned acc, const BwdWorkspace &ws,
                                   const float2 *rope, hipStream_t s)
{
    if (g.N() == 0) {   // no tokens: only dgates is written (zero), unless it accumulates
        if (acc & 4u) return hipSuccess;
        hipLaunchKernelGGL(fill_zero, dim3((unsigned)((4 * g.HD() + 255) / 256)), dim3(256), 0, s,
                           dgates, (int64_t)4 * g.HD());
        return hipGetLastError();
    }
    // 1. attention backward: dq, and the gradients of the mixed entries into dk/dv
    if (g.dtype == MAGLEV_BF16) {
        mfma::launch_attn_bwd_bf16(g, q, kx, vx, o, lse, dO, dq, dk, dv, ws, rope, true, s);
    } else if (g.Dh == 128) {
        attn_bwd_simt<float, 128, false, false>(g, q, kx, vx, nullptr, nullptr, nullptr, o, lse, dO,
                                                dq, dk, dv, ws, rope, s);
    } else {
        attn_bwd_simt<float, 64, false, false>(g, q, kx, vx, nullptr, nullptr, nullptr, o, lse, dO,
                                               dq, dk, dv, ws, rope, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 2. gates, rotation and norm backward: dk, dv final; this layer's share of
    // the shared projections' gradients written or added in float32
    return launch_gated_mix_bwd(g, k, v, kp, vm, gates, eps, rope, dk, dv, ws, dgates, acc, dkp,
                                dvm, s);
}

hipError_t launch_mem_project_bwd(const Geom &g, const float *dkm, const float *dvm,
                                  const void *m_prime, const void *wk, const void *wv,
                                  float *dm_prime, float *dWk, float *dWv, unsigned acc,
                                  const BwdWorkspace &ws, hipStream_t s)
{
    const int HD = g.HD();
    if (g.N() == 0) {
        const int64_t nw = (int64_t)HD * g.d;
        if (!(acc & 2u)) {
            hipLaunchKernelGGL(fill_zero, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, dWk, nw);
            hipLaunchKernelGGL(fill_zero, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, dWv, nw);
        }
        return hipGetLastError();
    }
    if (g.dtype == MAGLEV_BF16) {
        const int64_t n8 = g.N() * (int64_t)HD / 8;
        {
            prof::Scope ts("proj_bwd_to_bf16", s);
            hipLaunchKernelGGL(to_bf16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, dkm,
                               static_cast<bf16 *>(ws.dkp), n8);
            hipLaunchKernelGGL(to_bf16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, dvm,
                               static_cast<bf16 *>(ws.dvm), n8);
        }
        mfma::launch_proj_bwd_bf16(g, ws.dkp, ws.dvm, m_prime, wk, wv, nullptr, dm_prime, dWk, dWv,
                                   acc, ws, s);
        return hipGetLastError();
    }
    if (!(acc & 1u)) {
        prof::Scope ts("zero_last_rows", s);
        hipLaunchKernelGGL(zero_last_rows, dim3(g.B), dim3(256), 0, s, dm_prime, g.B, g.T, g.d);
    }
    proj_bwd_simt<float>(g, dkm, dvm, m_prime, wk, wv, nullptr, dm_prime, dWk, dWv, acc, s);
    return hipGetLastError();
}

}  // namespace maglev
