// loss_head.hip -- the loss head that closes the lifted pass: final RMSNorm of
// the decoder's last hidden state, the soft-capped LM head, the mean
// cross-entropy, the memory-consistency term, and the gradients.
//
// Method: Maglev summary on paper.rainbus.top ("Maglev：滑动窗口循环记忆"),
// section 方法步骤详情: the output state m_t feeds the LM head
// softmax(15 tanh(U m_t / 15)), and the loss averages CE + lambda
// ||m_t - m'_t||^2 / sqrt(d) over positions; the targets m' are states after
// the final RMSNorm, so m_t = RMSNorm(h_t) (no learned scale).
//   m_n  = h_n r_n,  r_n = 1 / sqrt(mean(h_n^2) + eps)
//   c_nv = cap tanh((U m_n)_v / cap),  CE_n = lse_n - c_n,target_n
//   dz_nv = (softmax(c_n)_v - [v = target_n]) (1 - (c_nv / cap)^2) / N
//   dm = dz U + consistency term,  dU (+)= dz^T m,  dh = r (dm - m mean(dm m))
// The capped logits are materialised in float32 ([N, V]) by the head GEMM's
// epilogue; one workgroup per row then forms lse, CE and dz (three passes
// with the per-row sums of exp(c) over each column tile; one workgroup per row
// then forms lse, CE and dz in one pass over the row; dz (activation dtype)
// is the A operand of the two gradient products.
#include "common.hpp"
#include "internal.hpp"
#include "mfma_kernels.hpp"
#include "profile.hpp"
#include "simt_kernels.hpp"

namespace maglev {

namespace {

// m = h r, rstd[n] = r: one wave per row, 8 elements a lane per step.
template <typename T>
__global__ __launch_bounds__(256) void head_norm(int64_t N, int d, float eps, const T *h, T *m,
                                                 float *rstd)
{
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (n >= N) return;
    const T *hr = h + n * d;
    float ss = 0.0f;
    for (int c = 8 * lane; c < d; c += 512) {
        float x[8];
        load8(hr + c, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    }
    const float r = rsqrtf(wave_sum(ss) / (float)d + eps);
    for (int c = 8 * lane; c < d; c += 512) {
        float x[8];
        load8(hr + c, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= r;
        store8(m + n * d + c, x);
    }
    if (lane == 0) rstd[n] = r;
}

// dh (+)= r (dm - m mean(dm m)), m = h r: one wave per row.
template <typename T>
__global__ __launch_bounds__(256) void head_norm_bwd(int64_t N, int d, const T *h,
                                                     const float *rstd, const float *dm, float *dh,
                                                     unsigned acc)
{
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (n >= N) return;
    const float r = rstd[n];
    float s = 0.0f;
    for (int c = 8 * lane; c < d; c += 512) {
        float x[8], g[8];
        load8(h + n * d + c, x);
        load8(dm + n * d + c, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += g[e] * x[e] * r;
    }
    const float mu = wave_sum(s) / (float)d;
    for (int c = 8 * lane; c < d; c += 512) {
        float x[8], g[8], o[8];
        load8(h + n * d + c, x);
        load8(dm + n * d + c, g);
        if (acc) load8(dh + n * d + c, o);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = r * (g[e] - x[e] * r * mu);
            o[e] = acc ? o[e] + v : v;
        }
        store8(dh + n * d + c, o);
    }
}

MAGLEV_DEV float block_total(float x, float *red)
{
    x = wave_sum(x);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// One workgroup (256 threads) per row n of the capped logits c [N, V]:
// lse_n = log sum_v exp(c_nv) (no running maximum: |c| <= cap <= 64 keeps
// every exp(c) finite and normal in float32), CE_n (0 for a target outside
// [0, V)), and, when dz is not null, dz[n, :] as above. The row's sum comes
// from the ntn per-tile partial sums the head product wrote (rowsum != null)
// or from a pass over the row. V is a multiple of 8.
template <typename T>
__global__ __launch_bounds__(256) void head_ce(int64_t N, int64_t V, float cap, const float *c,
                                               const float *rowsum, int64_t ntn,
                                               const int64_t *targets, float *ce, T *dz)
{
    __shared__ float red[4];
    const int64_t n = blockIdx.x;
    const float *row = c + n * V;
    float sum = 0.0f;
    if (rowsum) {
        for (int64_t t = threadIdx.x; t < ntn; t += 256) sum += rowsum[n * ntn + t];
    } else {
        for (int64_t v = 8 * (int64_t)threadIdx.x; v < V; v += 2048) {
            float x[8];
            load8(row + v, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += __expf(x[e]);
        }
    }
    sum = block_total(sum, red);
    const float lse = __logf(sum);
    const int64_t tgt = targets[n];
    const bool valid = tgt >= 0 && tgt < V;
    if (threadIdx.x == 0) ce[n] = valid ? lse - row[tgt] : 0.0f;
    if (!dz) return;
    const float inv_n = 1.0f / (float)N, inv_cap = 1.0f / cap;
    for (int64_t v = 8 * (int64_t)threadIdx.x; v < V; v += 2048) {
        float x[8];
        load8(row + v, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float t = x[e] * inv_cap;
            const float p = __expf(x[e] - lse) - (v + e == tgt ? 1.0f : 0.0f);
            x[e] = valid ? p * (1.0f - t * t) * inv_n : 0.0f;
        }
        store8(dz + n * V + v, x);
    }
}

// loss (+)= sum_n ce[n] / N, one workgroup, fixed order.
__global__ __launch_bounds__(256) void head_loss(int64_t N, const float *ce, float *loss,
                                                 unsigned acc)
{
    __shared__ float red[4];
    float s = 0.0f;
    for (int64_t i = threadIdx.x; i < N; i += 256) s += ce[i];
    s = block_total(s, red);
    if (threadIdx.x == 0) {
        const float v = s / (float)N;
        *loss = acc ? *loss + v : v;
    }
}

// float32 path: the three products on the tiled fp32 GEMM.
struct F32Rows {   // A(row, k) = x[row, k], stored [rows][ld]
    const float *x;
    int64_t ld;
    __device__ float operator()(int64_t r, int64_t k) const { return x[r * ld + k]; }
};
struct F32RowsT {  // B(k, n) = x[n, k] (a row-major matrix read transposed)
    const float *x;
    int64_t ld;
    __device__ float operator()(int64_t k, int64_t n) const { return x[n * ld + k]; }
};
struct F32ColsT {  // A(r, k) = x[k, r]
    const float *x;
    int64_t ld;
    __device__ float operator()(int64_t r, int64_t k) const { return x[k * ld + r]; }
};
struct CapStore {
    float *out;
    int64_t ld;
    float cap;
    __device__ void operator()(int64_t r, int64_t n, float x) const
    {
        out[r * ld + n] = cap * tanhf(x / cap);
    }
};
struct PlainStore {
    float *out;
    int64_t ld;
    bool acc;
    __device__ void operator()(int64_t r, int64_t n, float x) const
    {
        float *p = out + r * ld + n;
        *p = acc ? *p + x : x;
    }
};

}  // namespace

size_t lm_head_workspace_bytes(int64_t N, int d, int64_t V, int dtype, HeadWorkspace *L,
                               char *base)
{
    auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t esz = dtype == MAGLEV_BF16 ? 2 : 4;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align(off + bytes); return o; };
    const size_t oR = take((size_t)N * sizeof(float));
    const size_t oC = take((size_t)N * sizeof(float));
    const size_t oL = take((size_t)N * V * sizeof(float));
    const size_t oP = take((size_t)N * mfma::lm_logits_col_tiles(V) * sizeof(float));
    const size_t oZ = take((size_t)N * V * esz);
    const size_t oM = take((size_t)N * d * sizeof(float));
    const size_t oS = take(loss_workspace_bytes(N, d));
    const size_t oU = take(dtype == MAGLEV_BF16 ? (size_t)d * V * 2 : 0);
    L->rstd = base ? reinterpret_cast<float *>(base + oR) : nullptr;
    L->ce = base ? reinterpret_cast<float *>(base + oC) : nullptr;
    L->logits = base ? reinterpret_cast<float *>(base + oL) : nullptr;
    L->rowsum = base ? reinterpret_cast<float *>(base + oP) : nullptr;
    L->dz = base ? static_cast<void *>(base + oZ) : nullptr;
    L->dm = base ? reinterpret_cast<float *>(base + oM) : nullptr;
    L->loss_ws = base ? static_cast<void *>(base + oS) : nullptr;
    L->ut = base && dtype == MAGLEV_BF16 ? static_cast<void *>(base + oU) : nullptr;
    return off;
}

template <typename T>
static hipError_t lm_head_t(int64_t N, int d, int64_t V, float cap, float eps, float lambda,
                            int dtype, const void *hv, const void *Uv, const int64_t *targets,
                            const void *mpv, void *mv, float *loss, float *dh, float *dU,
                            unsigned acc, const HeadWorkspace &ws, hipStream_t s)
{
    const T *h = static_cast<const T *>(hv);
    T *m = static_cast<T *>(mv);
    const bool grads = dh || dU;
    {
        prof::Scope ts("head_norm", s);
        hipLaunchKernelGGL(head_norm<T>, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, N, d, eps,
                           h, m, ws.rstd);
    }
    if constexpr (sizeof(T) == 2) {
        mfma::launch_lm_logits_bf16(N, V, d, cap, m, Uv, ws.logits, ws.rowsum, s);
    } else {
        prof::Scope ts("lm_logits", s);
        simt::gemm_tiled<F32Rows, F32RowsT, CapStore><<<dim3((unsigned)((V + 63) / 64),
                                                               (unsigned)((N + 63) / 64)),
                                                          256, 0, s>>>(
            N, V, d, F32Rows{reinterpret_cast<const float *>(m), d},
            F32RowsT{static_cast<const float *>(Uv), d}, CapStore{ws.logits, V, cap});
    }
    {
        prof::Scope ts("head_ce", s);
        const bool sums = sizeof(T) == 2;   // the MFMA head product writes row sums
        hipLaunchKernelGGL(head_ce<T>, dim3((unsigned)N), dim3(256), 0, s, N, V, cap, ws.logits,
                           sums ? ws.rowsum : nullptr, mfma::lm_logits_col_tiles(V), targets,
                           ws.ce, grads ? static_cast<T *>(ws.dz) : nullptr);
        hipLaunchKernelGGL(head_loss, dim3(1), dim3(256), 0, s, N, ws.ce, loss, acc & 4u);
    }
    if (grads) {
        if constexpr (sizeof(T) == 2) {
            mfma::launch_lm_dm_bf16(N, V, d, ws.dz, Uv, ws.ut, ws.dm, s);
            if (dU) mfma::launch_lm_du_bf16(N, V, d, ws.dz, m, dU, (acc & 2u) != 0, s);
        } else {
            const float *dz = static_cast<const float *>(ws.dz);
            {
                prof::Scope ts("lm_dm", s);
                simt::gemm_tiled<F32Rows, F32Rows, PlainStore><<<dim3((unsigned)((d + 63) / 64),
                                                                      (unsigned)((N + 63) / 64)),
                                                                 256, 0, s>>>(
                    N, d, V, F32Rows{dz, V}, F32Rows{static_cast<const float *>(Uv), d},
                    PlainStore{ws.dm, d, false});
            }
            if (dU) {
                prof::Scope ts("lm_du", s);
                simt::gemm_tiled<F32ColsT, F32Rows, PlainStore><<<dim3((unsigned)((d + 63) / 64),
                                                                       (unsigned)((V + 63) / 64)),
                                                                  256, 0, s>>>(
                    V, d, N, F32ColsT{dz, V}, F32Rows{reinterpret_cast<const float *>(m), d},
                    PlainStore{dU, d, (acc & 2u) != 0});
            }
        }
    }
    // the consistency term on m = RMSNorm(h): loss +=, and dm += its gradient
    if (mpv) {
        hipError_t e = launch_loss(N, d, lambda, dtype, m, mpv, loss, grads ? ws.dm : nullptr,
                                   nullptr, 4u | 1u, ws.loss_ws, s);
        if (e != hipSuccess) return e;
    }
    if (dh) {
        prof::Scope ts("head_norm_bwd", s);
        hipLaunchKernelGGL(head_norm_bwd<T>, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, N, d,
                           h, ws.rstd, ws.dm, dh, acc & 1u);
    }
    return hipGetLastError();
}

hipError_t launch_lm_head(int64_t N, int d, int64_t V, float cap, float eps, float lambda,
                          int dtype, const void *h, const void *U, const int64_t *targets,
                          const void *m_prime, void *m, float *loss, float *dh, float *dU,
                          unsigned acc, const HeadWorkspace &ws, hipStream_t s)
{
    if (dtype == MAGLEV_BF16)
        return lm_head_t<bf16>(N, d, V, cap, eps, lambda, dtype, h, U, targets, m_prime, m, loss,
                               dh, dU, acc, ws, s);
    return lm_head_t<float>(N, d, V, cap, eps, lambda, dtype, h, U, targets, m_prime, m, loss, dh,
                            dU, acc, ws, s);
}

}  // namespace maglev
