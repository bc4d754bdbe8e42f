// simt_kernels.hpp -- straightforward vector-ALU kernels of the attention path:
// one workgroup per row with one thread per channel, and a tiled fp32 GEMM
// driven by element accessors. They are the float32 path (exact algebra in
// fp32, used by the fp32 workloads) and the structural template the MFMA
// kernels are checked against. Storage type T is float or bf16; arithmetic
// is float32.
//
// Method: Maglev summary on paper.rainbus.top ("Maglev：滑动窗口循环记忆"),
// sections 前置知识 (SWA window, RoPE on local and injected keys) and
// 方法步骤详情 (shifted memory m'_{0:T-1} with m'_0 = 0, projection to K/V
// features, gated mix, attention over the W most recent mixed entries).
#pragma once

#include "common.hpp"

namespace maglev {
namespace simt {

// Sum over the workgroup (blockDim.x = NT threads, NT in {64, 128}); every
// thread receives the total. red must hold NT/64 floats.
template <int NT>
MAGLEV_DEV float block_sum(float x, float *red)
{
    x = wave_sum(x);
    if constexpr (NT == 64) {
        return x;
    } else {
        const int w = threadIdx.x >> 6;
        __syncthreads();
        if ((threadIdx.x & 63) == 0) red[w] = x;
        __syncthreads();
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < NT / 64; ++i) t += red[i];
        return t;
    }
}

// Rotated value of channel c of row x at table row `tab` (nullptr: no RoPE).
// Channel c pairs with c + Dh/2 (half-split pairing).
template <typename T, int DH>
MAGLEV_DEV float rope_channel(const T *x, int c, const float2 *tab, bool inverse)
{
    const float a = to_f<T>(x[c]);
    if (!tab) return a;
    constexpr int half = DH / 2;
    const int i = c < half ? c : c - half;
    const float2 cs = tab[i];
    const float sn = inverse ? -cs.y : cs.y;
    if (c < half) return a * cs.x - to_f<T>(x[c + half]) * sn;
    return to_f<T>(x[c - half]) * sn + a * cs.x;
}

// Same for a float row held in shared memory.
template <int DH>
MAGLEV_DEV float rope_channel_f(const float *x, int c, const float2 *tab, bool inverse)
{
    const float a = x[c];
    if (!tab) return a;
    constexpr int half = DH / 2;
    const int i = c < half ? c : c - half;
    const float2 cs = tab[i];
    const float sn = inverse ? -cs.y : cs.y;
    if (c < half) return a * cs.x - x[c + half] * sn;
    return x[c - half] * sn + a * cs.x;
}

struct RowArgs {
    int64_t B, T;
    int H, W;
    int64_t pos0;
    float scale;
    const float2 *rope;   // [pos][Dh/2] or nullptr
    const float *gate;    // [H] logits
};

MAGLEV_DEV const float2 *rope_row(const RowArgs &a, int64_t t, int Dh)
{
    return a.rope ? a.rope + (a.pos0 + t) * (Dh / 2) : nullptr;
}

// ---------------------------------------------------------------------------
// Forward: one workgroup per (i, h, b), one thread per channel.
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ __launch_bounds__(DH) void attn_fwd_rows(RowArgs a, const T *q, const T *kx,
                                                     const T *vx, T *o, float *lse)
{
    __shared__ float red[2];
    const int64_t i = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int c = threadIdx.x;
    const int64_t qrow = (b * a.T + i) * a.H + h;
    const float qh = rope_channel<T, DH>(q + qrow * DH, c, rope_row(a, i, DH), false);
    const int64_t lo = i - a.W + 1 > 0 ? i - a.W + 1 : 0;
    float mx = -INFINITY, l = 0.0f, acc = 0.0f;
    for (int64_t j = lo; j <= i; ++j) {
        const int64_t krow = (b * a.T + j) * a.H + h;
        const float kt = to_f<T>(kx[krow * DH + c]), vt = to_f<T>(vx[krow * DH + c]);
        const float sc = block_sum<DH>(qh * kt, red) * a.scale;
        const float mn = fmaxf(mx, sc);
        const float corr = __expf(mx - mn);
        const float p = __expf(sc - mn);
        l = l * corr + p;
        acc = acc * corr + p * vt;
        mx = mn;
    }
    o[qrow * DH + c] = from_f<T>(acc / l);
    if (lse && c == 0) lse[(b * a.H + h) * a.T + i] = mx + __logf(l);
}

// D_i = sum_c dO_ic O_ic.
template <typename T, int DH>
__global__ __launch_bounds__(DH) void bwd_rowdot(RowArgs a, const T *o, const T *dO, float *D)
{
    __shared__ float red[2];
    const int64_t i = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int c = threadIdx.x;
    const int64_t row = (b * a.T + i) * a.H + h;
    const float x = block_sum<DH>(to_f<T>(o[row * DH + c]) * to_f<T>(dO[row * DH + c]), red);
    if (c == 0) D[(b * a.H + h) * a.T + i] = x;
}

// dq: one workgroup per query row.
//   P_ij = exp(scale q^_i.k~_j - lse_i), dP_ij = dO_i.v~_j, dS_ij = P_ij (dP_ij - D_i),
//   dq^_i = scale sum_j dS_ij k~_j, dq_i = R_i^T dq^_i.
template <typename T, int DH>
__global__ __launch_bounds__(DH) void bwd_dq_rows(RowArgs a, const T *q, const T *kx, const T *vx,
                                                   const T *dO, const float *lse, const float *D,
                                                   T *dq)
{
    __shared__ float red[2];
    __shared__ float dqh[DH];
    const int64_t i = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int c = threadIdx.x;
    const int64_t qrow = (b * a.T + i) * a.H + h;
    const float2 *tab_i = rope_row(a, i, DH);
    const float qh = rope_channel<T, DH>(q + qrow * DH, c, tab_i, false);
    const float dOi = to_f<T>(dO[qrow * DH + c]);
    const float li = lse[(b * a.H + h) * a.T + i];
    const float Di = D[(b * a.H + h) * a.T + i];
    const int64_t lo = i - a.W + 1 > 0 ? i - a.W + 1 : 0;
    float acc = 0.0f;
    for (int64_t j = lo; j <= i; ++j) {
        const int64_t krow = (b * a.T + j) * a.H + h;
        const float kt = to_f<T>(kx[krow * DH + c]), vt = to_f<T>(vx[krow * DH + c]);
        const float sc = block_sum<DH>(qh * kt, red) * a.scale;
        const float dp = block_sum<DH>(dOi * vt, red);
        const float p = __expf(sc - li);
        acc += p * (dp - Di) * kt;
    }
    dqh[c] = acc * a.scale;
    __syncthreads();
    dq[qrow * DH + c] = from_f<T>(rope_channel_f<DH>(dqh, c, tab_i, true));
}

// dk, dv: one workgroup per key row j; queries i in [j, j+W-1]; k~ = kx, v~ = vx.
//   dk~_j = scale sum_i dS_ij q^_i, dv~_j = sum_i P_ij dO_i,
//   dk_j = R_j^T dk~_j, dv_j = dv~_j,
//   ds_part[b,h,j] = <kmem_j, dk_j> + <vmem_j, dv_j>  (d loss / d s_h, this key).
// ROTATE false: write dk~_j itself (rotated frame) instead of dk_j.
// PARTIAL false: no gate partial (km, vm, ds_part are not read or written).
template <typename T, int DH, bool ROTATE, bool PARTIAL>
__global__ __launch_bounds__(DH) void bwd_dkdv_rows(RowArgs a, const T *q, const T *kx,
                                                     const T *vx, const T *km, const T *vm,
                                                     const T *dO, const float *lse, const float *D,
                                                     T *dk, T *dv, float *ds_part)
{
    __shared__ float red[2];
    __shared__ float dkt[DH];
    const int64_t j = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int c = threadIdx.x;
    const int64_t krow = (b * a.T + j) * a.H + h;
    const float kt = to_f<T>(kx[krow * DH + c]), vt = to_f<T>(vx[krow * DH + c]);
    const int64_t hi = j + a.W - 1 < a.T - 1 ? j + a.W - 1 : a.T - 1;
    float acck = 0.0f, accv = 0.0f;
    for (int64_t i = j; i <= hi; ++i) {
        const int64_t qrow = (b * a.T + i) * a.H + h;
        const float qh = rope_channel<T, DH>(q + qrow * DH, c, rope_row(a, i, DH), false);
        const float dOi = to_f<T>(dO[qrow * DH + c]);
        const float sc = block_sum<DH>(qh * kt, red) * a.scale;
        const float dp = block_sum<DH>(dOi * vt, red);
        const float p = __expf(sc - lse[(b * a.H + h) * a.T + i]);
        const float ds = p * (dp - D[(b * a.H + h) * a.T + i]);
        acck += ds * qh;
        accv += p * dOi;
    }
    if constexpr (!ROTATE) {
        dk[krow * DH + c] = from_f<T>(acck * a.scale);
        dv[krow * DH + c] = from_f<T>(accv);
        return;
    }
    dkt[c] = acck * a.scale;
    __syncthreads();
    const float dkc = rope_channel_f<DH>(dkt, c, rope_row(a, j, DH), true);
    dk[krow * DH + c] = from_f<T>(dkc);
    dv[krow * DH + c] = from_f<T>(accv);
    if constexpr (!PARTIAL) return;
    const float part = dkc * to_f<T>(km[krow * DH + c]) + accv * to_f<T>(vm[krow * DH + c]);
    const float tot = block_sum<DH>(part, red);
    if (c == 0) ds_part[(b * a.H + h) * a.T + j] = tot;
}

// ---------------------------------------------------------------------------
// Gated mix, one 8-channel chunk pair (c, c + Dh/2) per thread:
//   kmix = R_p (k + s_h kmem),  vmix = v + s_h vmem,  p = pos0 + t.
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ __launch_bounds__(256) void mix_entries(int64_t rows, int H, int64_t Tlen, int64_t pos0,
                                                   const float2 *rope, const float *gate,
                                                   const T *k, const T *v, const T *km,
                                                   const T *vm, T *kx, T *vx)
{
    constexpr int CP = DH / 16;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / CP;            // (b*T + t)*H + h
    if (row >= rows) return;
    const int cc = (int)(gid % CP);
    const int h = (int)(row % H);
    const int64_t t = (row / H) % Tlen;
    const float s = gate_sigmoid(gate[h]);
    const int64_t base = row * DH + 8 * cc;
    float lo[8], hi[8], mlo[8], mhi[8];
    load8(k + base, lo);
    load8(k + base + DH / 2, hi);
    load8(km + base, mlo);
    load8(km + base + DH / 2, mhi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e] += s * mlo[e];
        hi[e] += s * mhi[e];
    }
    if (rope) {
        const float2 *cs = rope + (pos0 + t) * (DH / 2) + 8 * cc;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float c = cs[e].x, sn = cs[e].y, x0 = lo[e], x1 = hi[e];
            lo[e] = x0 * c - x1 * sn;
            hi[e] = x0 * sn + x1 * c;
        }
    }
    store8(kx + base, lo);
    store8(kx + base + DH / 2, hi);
    load8(v + base, lo);
    load8(v + base + DH / 2, hi);
    load8(vm + base, mlo);
    load8(vm + base + DH / 2, mhi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e] += s * mlo[e];
        hi[e] += s * mhi[e];
    }
    store8(vx + base, lo);
    store8(vx + base + DH / 2, hi);
}

// ---------------------------------------------------------------------------
// Rotated keys of attention without injection: kr = R_p k, p = pos0 + t, one
// 8-channel chunk pair (c, c + Dh/2) per thread.
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ __launch_bounds__(256) void rope_rows(int64_t rows, int H, int64_t Tlen, int64_t pos0,
                                                 const float2 *rope, const T *k, T *kr)
{
    constexpr int CP = DH / 16;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / CP;            // (b*T + t)*H + h
    if (row >= rows) return;
    const int cc = (int)(gid % CP);
    const int64_t t = (row / H) % Tlen;
    const int64_t base = row * DH + 8 * cc;
    float lo[8], hi[8];
    load8(k + base, lo);
    load8(k + base + DH / 2, hi);
    if (rope) {
        const float2 *cs = rope + (pos0 + t) * (DH / 2) + 8 * cc;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float c = cs[e].x, sn = cs[e].y, x0 = lo[e], x1 = hi[e];
            lo[e] = x0 * c - x1 * sn;
            hi[e] = x0 * sn + x1 * c;
        }
    }
    store8(kr + base, lo);
    store8(kr + base + DH / 2, hi);
}

// ---------------------------------------------------------------------------
// Tiled fp32 GEMM: C(m, n) = sum_k A(m, k) B(k, n), 64x64 tile, 4x4 per thread.
// LA/LB return operands as float (0 outside the matrix); ST stores a result.
// ---------------------------------------------------------------------------
template <class LA, class LB, class ST>
__global__ __launch_bounds__(256) void gemm_tiled(int64_t M, int64_t N, int64_t K, LA la, LB lb,
                                                  ST st)
{
    __shared__ float As[16][65];
    __shared__ float Bs[16][65];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += 16) {
        for (int e = threadIdx.x; e < 16 * 64; e += 256) {
            const int kk = e >> 6, xx = e & 63;
            const int64_t kg = k0 + kk;
            As[kk][xx] = (kg < K && m0 + xx < M) ? la(m0 + xx, kg) : 0.0f;
            Bs[kk][xx] = (kg < K && n0 + xx < N) ? lb(kg, n0 + xx) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float av[4], bv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) av[r] = As[kk][ty * 4 + r];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) bv[cc] = Bs[kk][tx * 4 + cc];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) acc[r][cc] += av[r] * bv[cc];
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int64_t m = m0 + ty * 4 + r, n = n0 + tx * 4 + cc;
            if (m < M && n < N) st(m, n, acc[r][cc]);
        }
}

}  // namespace simt
}  // namespace maglev
