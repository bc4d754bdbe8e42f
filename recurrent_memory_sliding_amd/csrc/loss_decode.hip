// loss_decode.hip -- memory-bound kernels: the memory-consistency loss and the
// recurrent decode step on a W-slot ring cache (plus the position advance).
//
// Loss: Maglev summary on paper.rainbus.top ("Maglev：滑动窗口循环记忆"),
// sections 核心方法 and 方法步骤详情: lambda * ||m_t - m'_t||^2 / sqrt(d),
// averaged over the positions.
// Decode: same page, section 方法步骤详情 (recurrent inference
// m_t = P(x_{t-W+1:t}, M_{t-1})) and section 前置知识 (KV cache; the memory rides
// in the existing entries); gist.science summary ("Technische Samenvatting:
// Maglev - Sliding Recurrent Memory"), section Inferentiemechanisme.
#include "common.hpp"
#include "internal.hpp"
#include "profile.hpp"

namespace maglev {

// ============================================================================
// Consistency loss
// ============================================================================
constexpr int kLossThreads = 256;
constexpr int kLossMaxBlocks = 2048;

static int loss_blocks(int64_t n8)
{
    int64_t nb = (n8 + kLossThreads - 1) / kLossThreads;
    if (nb < 1) nb = 1;
    if (nb > kLossMaxBlocks) nb = kLossMaxBlocks;
    return (int)nb;
}

size_t loss_workspace_bytes(int64_t, int) { return kLossMaxBlocks * sizeof(float); }

// Each thread walks a fixed grid-stride sequence of 8-element chunks, so the
// partial sums (and the final reduction order) depend only on (N, d).
template <typename T>
__global__ __launch_bounds__(kLossThreads) void loss_partial(int64_t n8, const T *m, const T *mp,
                                                             float g2, float *dm, float *dmp,
                                                             unsigned acc, float *partial)
{
    __shared__ float red[kLossThreads / 64];
    float sum = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * kLossThreads;
    for (int64_t i = (int64_t)blockIdx.x * kLossThreads + threadIdx.x; i < n8; i += stride) {
        float a[8], b[8], g[8];
        load8(m + 8 * i, a);
        load8(mp + 8 * i, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float diff = a[e] - b[e];
            sum += diff * diff;
            g[e] = g2 * diff;
        }
        if (dm) {
            float out[8];
            if (acc & 1u) load8(dm + 8 * i, out);
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = (acc & 1u) ? out[e] + g[e] : g[e];
            store8(dm + 8 * i, out);
        }
        if (dmp) {
            float out[8];
            if (acc & 2u) load8(dmp + 8 * i, out);
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = (acc & 2u) ? out[e] - g[e] : -g[e];
            store8(dmp + 8 * i, out);
        }
    }
    sum = wave_sum(sum);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < kLossThreads / 64; ++w) t += red[w];
        partial[blockIdx.x] = t;
    }
}

__global__ __launch_bounds__(1024) void loss_final(const float *partial, int n, float c,
                                                   float *loss, unsigned acc)
{
    __shared__ float red[16];
    float t = 0.0f;
    for (int i = threadIdx.x; i < n; i += 1024) t += partial[i];
    t = wave_sum(t);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = 0.0f;
        for (int w = 0; w < 16; ++w) s += red[w];
        const float l = c * s;
        *loss = (acc & 4u) ? *loss + l : l;
    }
}

hipError_t launch_loss(int64_t N, int d, float lambda, int dtype, const void *m, const void *mp,
                       float *loss, float *dm, float *dmp, unsigned acc, void *ws, hipStream_t s)
{
    const int64_t n8 = N * (int64_t)d / 8;
    const float c = N > 0 ? (float)((double)lambda / ((double)N * sqrt((double)d))) : 0.0f;
    const int nb = loss_blocks(n8);
    float *partial = static_cast<float *>(ws);
    {
    prof::Scope ts("loss_partial", s);
    if (dtype == MAGLEV_BF16)
        hipLaunchKernelGGL(loss_partial<bf16>, dim3(nb), dim3(kLossThreads), 0, s, n8,
                           static_cast<const bf16 *>(m), static_cast<const bf16 *>(mp), 2.0f * c,
                           dm, dmp, acc, partial);
    else
        hipLaunchKernelGGL(loss_partial<float>, dim3(nb), dim3(kLossThreads), 0, s, n8,
                           static_cast<const float *>(m), static_cast<const float *>(mp), 2.0f * c,
                           dm, dmp, acc, partial);
    }
    prof::Scope ts("loss_final", s);
    hipLaunchKernelGGL(loss_final, dim3(1), dim3(1024), 0, s, partial, nb, c, loss, acc);
    return hipGetLastError();
}

// ============================================================================
// Decode step
// ============================================================================
// Work split: every (stream b, head h) ring of W slots is cut into chunks of
// kSlotsPerSplit slots; one workgroup per (chunk, h, b) computes a partial
// softmax state (running max, sum, unnormalised output) into the workspace,
// and a combine kernel merges the chunks. Only the chunk that owns slot
// p mod W writes the new entry; it also uses the new entry from shared memory,
// so no workgroup reads a ring slot another workgroup writes.
constexpr int kSlotsPerSplit = 64;
constexpr int kDecThreads = 256;

static int decode_splits(int W) { return (W + kSlotsPerSplit - 1) / kSlotsPerSplit; }

size_t decode_workspace_bytes(int Bs, int H, int Dh, int W)
{
    return (size_t)Bs * H * decode_splits(W) * (Dh + 4) * sizeof(float);
}

// p - ((p - s) mod W) >= 0  <=>  slot s has been written at or before position p.
MAGLEV_DEV bool slot_valid(int64_t p, int64_t s, int W)
{
    int64_t back = (p - s) % W;
    if (back < 0) back += W;
    return p - back >= 0;
}

template <typename T, int DH>
__global__ __launch_bounds__(kDecThreads) void decode_partial(
    int H, int W, float rope_base, float scale, const T *q, const T *k, const T *v, const T *km,
    const T *vm, const float *gate, T *kcache, T *vcache, const int64_t *pos, float *ws)
{
    constexpr int CH = DH / 8;                 // 8-element chunks per row
    constexpr int ROWS = kDecThreads / CH;     // slots per pass
    constexpr int PASSES = kSlotsPerSplit / ROWS;
    __shared__ float qh[DH];
    __shared__ float knew[DH], vnew[DH];
    __shared__ float sc[kSlotsPerSplit];
    __shared__ float opart[ROWS][DH + 4];

    const int split = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int nsplit = gridDim.x;
    const int tid = threadIdx.x;
    const int64_t p = pos[b];
    const int slot_new = (int)(p % W);
    const int s0 = split * kSlotsPerSplit;
    const int s1 = min(W, s0 + kSlotsPerSplit);
    const bool owns_new = slot_new >= s0 && slot_new < s1;
    const int64_t row = b * H + h;                  // [Bs,H,*] row
    const float sg = gate_sigmoid(gate[h]);

    // Rotation of position p, evaluated in double precision (exact enough for
    // any position; no table bound).
    if (tid < DH / 2) {
        const int i = tid;
        float cs = 1.0f, sn = 0.0f;
        if (rope_base > 0.0f) {
            const double theta = pow((double)rope_base, -2.0 * (double)i / (double)DH);
            double sd, cd;
            sincos((double)p * theta, &sd, &cd);
            cs = (float)cd;
            sn = (float)sd;
        }
        const T *qr = q + row * DH;
        const float a0 = to_f<T>(qr[i]), a1 = to_f<T>(qr[i + DH / 2]);
        const float ls = scale * kLog2e;
        qh[i] = (a0 * cs - a1 * sn) * ls;
        qh[i + DH / 2] = (a0 * sn + a1 * cs) * ls;
        if (owns_new) {
            const T *kr = k + row * DH, *kmr = km + row * DH;
            const float x0 = to_f<T>(kr[i]) + sg * to_f<T>(kmr[i]);
            const float x1 = to_f<T>(kr[i + DH / 2]) + sg * to_f<T>(kmr[i + DH / 2]);
            const T k0 = from_f<T>(x0 * cs - x1 * sn);
            const T k1 = from_f<T>(x0 * sn + x1 * cs);
            const T v0 = from_f<T>(to_f<T>(v[row * DH + i]) + sg * to_f<T>(vm[row * DH + i]));
            const T v1 = from_f<T>(to_f<T>(v[row * DH + i + DH / 2]) +
                                   sg * to_f<T>(vm[row * DH + i + DH / 2]));
            T *kc = kcache + (row * W + slot_new) * DH;
            T *vc = vcache + (row * W + slot_new) * DH;
            kc[i] = k0; kc[i + DH / 2] = k1;
            vc[i] = v0; vc[i + DH / 2] = v1;
            knew[i] = to_f<T>(k0); knew[i + DH / 2] = to_f<T>(k1);
            vnew[i] = to_f<T>(v0); vnew[i + DH / 2] = to_f<T>(v1);
        }
    }
    __syncthreads();

    const int r = tid / CH, ch = tid % CH;
    float qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = qh[ch * 8 + e];

    // Issue every K and V load of this thread before using any of them.
    float kv[PASSES][8], vv[PASSES][8];
    bool ok[PASSES];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int sl = s0 + ps * ROWS + r;
        ok[ps] = sl < s1 && slot_valid(p, sl, W);
        if (ok[ps] && sl != slot_new) {
            load8(kcache + (row * W + sl) * DH + ch * 8, kv[ps]);
            load8(vcache + (row * W + sl) * DH + ch * 8, vv[ps]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kv[ps][e] = ok[ps] ? knew[ch * 8 + e] : 0.0f;
                vv[ps][e] = ok[ps] ? vnew[ch * 8 + e] : 0.0f;
            }
        }
    }
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d += qv[e] * kv[ps][e];
#pragma unroll
        for (int o = CH / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, 64);
        if (ch == 0) sc[ps * ROWS + r] = ok[ps] ? d : -INFINITY;
    }
    __syncthreads();
    float mx = -INFINITY;
    for (int i = 0; i < kSlotsPerSplit; ++i) mx = fmaxf(mx, sc[i]);
    float acc[8] = {};
    float lsum = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const float pr = ok[ps] ? exp2f(sc[ps * ROWS + r] - mx) : 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += pr * vv[ps][e];
        }
        for (int i = 0; i < kSlotsPerSplit; ++i) lsum += (sc[i] == -INFINITY) ? 0.0f : exp2f(sc[i] - mx);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) opart[r][ch * 8 + e] = acc[e];
    __syncthreads();
    float *out = ws + ((row * nsplit) + split) * (DH + 4);
    if (tid < DH) {
        float t = 0.0f;
#pragma unroll
        for (int rr = 0; rr < ROWS; ++rr) t += opart[rr][tid];
        out[4 + tid] = t;
    }
    if (tid == 0) {
        out[0] = mx;
        out[1] = lsum;
    }
}

template <typename T, int DH>
__global__ __launch_bounds__(DH) void decode_combine(int H, int nsplit, const float *ws, T *o)
{
    const int h = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t row = b * H + h;
    const float *base = ws + row * nsplit * (DH + 4);
    float mx = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, base[s * (DH + 4)]);
    float l = 0.0f, acc = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
        const float ms = base[s * (DH + 4)];
        if (ms == -INFINITY) continue;
        const float f = exp2f(ms - mx);
        l += f * base[s * (DH + 4) + 1];
        acc += f * base[s * (DH + 4) + 4 + threadIdx.x];
    }
    o[row * DH + threadIdx.x] = from_f<T>(acc / l);
}

template <typename T, int DH>
static void launch_decode_t(int Bs, int H, int W, float rope_base, float scale, const void *q,
                            const void *k, const void *v, const void *km, const void *vm,
                            const float *gate, void *kc, void *vc, const int64_t *pos, void *o,
                            void *ws, hipStream_t s)
{
    const int ns = decode_splits(W);
    {
    prof::Scope ts("decode_partial", s);
    hipLaunchKernelGGL((decode_partial<T, DH>), dim3(ns, H, Bs), dim3(kDecThreads), 0, s, H, W,
                       rope_base, scale, static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), static_cast<const T *>(km),
                       static_cast<const T *>(vm), gate, static_cast<T *>(kc),
                       static_cast<T *>(vc), pos, static_cast<float *>(ws));
    }
    prof::Scope ts("decode_combine", s);
    hipLaunchKernelGGL((decode_combine<T, DH>), dim3(H, Bs), dim3(DH), 0, s, H, ns,
                       static_cast<const float *>(ws), static_cast<T *>(o));
}

hipError_t launch_decode(int Bs, int H, int Dh, int W, float rope_base, float scale, int dtype,
                         const void *q, const void *k, const void *v, const void *km,
                         const void *vm, const float *gate, void *kc, void *vc,
                         const int64_t *pos, void *o, void *ws, hipStream_t s)
{
    if (dtype == MAGLEV_BF16) {
        if (Dh == 128)
            launch_decode_t<bf16, 128>(Bs, H, W, rope_base, scale, q, k, v, km, vm, gate, kc, vc, pos, o, ws, s);
        else
            launch_decode_t<bf16, 64>(Bs, H, W, rope_base, scale, q, k, v, km, vm, gate, kc, vc, pos, o, ws, s);
    } else {
        if (Dh == 128)
            launch_decode_t<float, 128>(Bs, H, W, rope_base, scale, q, k, v, km, vm, gate, kc, vc, pos, o, ws, s);
        else
            launch_decode_t<float, 64>(Bs, H, W, rope_base, scale, q, k, v, km, vm, gate, kc, vc, pos, o, ws, s);
    }
    return hipGetLastError();
}

__global__ void advance_pos(int Bs, int64_t *pos)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < Bs) pos[i] += 1;
}

hipError_t launch_advance(int Bs, int64_t *pos, hipStream_t s)
{
    hipLaunchKernelGGL(advance_pos, dim3((Bs + 255) / 256), dim3(256), 0, s, Bs, pos);
    return hipGetLastError();
}

}  // namespace maglev
