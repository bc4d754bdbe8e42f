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
#include <mutex>

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
        // every load of the chunk is issued before its first store (the
        // compiler cannot move a load across a store it cannot prove apart)
        float a[8], b[8], g[8], om[8], op[8];
        load8(m + 8 * i, a);
        load8(mp + 8 * i, b);
        if (dm && (acc & 1u)) load8(dm + 8 * i, om);
        if (dmp && (acc & 2u)) load8(dmp + 8 * i, op);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float diff = a[e] - b[e];
            sum += diff * diff;
            g[e] = g2 * diff;
        }
        if (dm) {
#pragma unroll
            for (int e = 0; e < 8; ++e) om[e] = (acc & 1u) ? om[e] + g[e] : g[e];
            store8(dm + 8 * i, om);
        }
        if (dmp) {
#pragma unroll
            for (int e = 0; e < 8; ++e) op[e] = (acc & 2u) ? op[e] - g[e] : -g[e];
            store8(dmp + 8 * i, op);
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
// Allocation-free consistency loss: the partial sums in a device array
// ============================================================================
// The partial sums of the allocation-free entry point (kLossMaxBlocks floats,
// 8 KB: the grid never has more workgroups, whatever N and d) live in this
// file-scope array, one copy per GPU for the life of the process. In host
// code the name `scratch` is a host-side stand-in, not the device address:
// the address is looked up once per device, with that device current, and
// only that address is handed to kernels. Every call on one GPU shares the
// array, so calls that overlap in time on one GPU race; each call writes
// every partial it reads, so nothing needs clearing between calls.
static __device__ __align__(256) float scratch[kLossMaxBlocks];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_addr[kScratchDevices] = {};   // per device: the address of `scratch` there
}  // namespace

size_t loss_scratch_bytes() { return sizeof(scratch); }

hipError_t loss_scratch_address(float **addr)
{
    *addr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_addr[dev] = static_cast<float *>(p);
    }
    *addr = g_scratch_addr[dev];
    return hipSuccess;
}

// ============================================================================
// Decode step
// ============================================================================
// One workgroup of 4 waves per (stream b, head h) covers the whole ring, so no
// cross-workgroup merge is needed and every workgroup of a 64-stream x
// 10-head step is resident at once (3 per CU fit). A slot row of Dh channels
// is read by Dh/8 lanes with 16-byte loads, so each wave instruction reads
// 64/(Dh/8) consecutive slots contiguously. The ring is cut into batches of
// kBatchPasses wave passes; batch j goes to wave j mod 4, which keeps an
// online softmax state per lane group and kDecBuffers batches in flight. The
// loads of a wave's first batches do not depend on the position (the slot
// about to be overwritten is read and discarded), so they are issued before
// pos[b] arrives and before the rotation of the new position is evaluated.
constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kBatchPasses = 4;
constexpr int kDecBuffers = 2;   // batches in flight per wave

size_t decode_workspace_bytes(int, int, int, int) { return 0; }

// Eight ring elements held as loaded (converted to float only when used).
// The rings are read once per step and every layer has its own (gigabytes in
// all, far more than the MALL holds), so the loads are nontemporal: on the
// chip this pattern streams at 5.9 TB/s with them against 5.3 TB/s without.
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
    u32x4 x;
    MAGLEV_DEV void load(const bf16 *p)
    {
        x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    }
    MAGLEV_DEV void get(float *out) const
    {
        const bf16x8 v = __builtin_bit_cast(bf16x8, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
    }
};
template <> struct Raw8<float> {
    f32x4 a, b;
    MAGLEV_DEV void load(const float *p)
    {
        a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        b = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + 4));
    }
    MAGLEV_DEV void get(float *out) const
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
    }
};

// Sum over aligned groups of N = 8 or 16 lanes, every lane of a group
// receiving it, with DPP moves inside 16-lane rows (no LDS-unit swizzles):
// partner 1 and 2 by quad permutation, then the mirror inside each half row
// (lane i and 7 - i), and for 16 lanes the mirror inside the row (i, 15 - i).
template <int N>
MAGLEV_DEV float group_sum_dpp(float x)
{
    static_assert(N == 8 || N == 16, "8- or 16-lane groups");
    auto add = [](float v, auto ctrl) {
        const int m = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), decltype(ctrl)::value,
                                                  0xF, 0xF, false);
        return v + __builtin_bit_cast(float, m);
    };
    x = add(x, std::integral_constant<int, 0xB1>{});    // quad_perm [1, 0, 3, 2]
    x = add(x, std::integral_constant<int, 0x4E>{});    // quad_perm [2, 3, 0, 1]
    x = add(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
    if constexpr (N == 16) x = add(x, std::integral_constant<int, 0x140>{});   // row_mirror
    return x;
}

// Merge softmax state (m2, l2, a2) into (m, l, a); -inf max marks an empty state.
template <int N>
MAGLEV_DEV void merge_state(float &m, float &l, float *a, float m2, float l2, const float *a2)
{
    const float mn = fmaxf(m, m2);
    const float f1 = m == -INFINITY ? 0.0f : exp2f(m - mn);
    const float f2 = m2 == -INFINITY ? 0.0f : exp2f(m2 - mn);
    m = mn;
    l = l * f1 + l2 * f2;
#pragma unroll
    for (int e = 0; e < N; ++e) a[e] = a[e] * f1 + a2[e] * f2;
}

// GATED = false: k~ = R_p (k + s_h kmem), v~ = v + s_h vmem, s_h = sigmoid(gate[h]).
// GATED = true:  k~ = g_kl R_p k + g_kr R_p RMSNorm(kmem), v~ = g_vl v + g_vr vmem,
//   g = 2 sigmoid(gates[..]) per channel of the H*Dh row, the norm over stream
//   b's whole H*Dh projection row (every workgroup of the stream recomputes it).
template <typename T, int DH, bool GATED>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    int H, int W, float rope_base, double log2_base, float scale, const T *q, const T *k,
    const T *v, const T *km, const T *vm, int64_t mem_stride, const float *gate,
    const float *gates, float eps, T *kcache, T *vcache, const int64_t *pos, T *o)
{
    constexpr int CH = DH / 8;                   // lanes per slot row
    constexpr int G = 64 / CH;                   // slots per wave pass
    constexpr int SB = G * kBatchPasses;         // slots per batch
    __shared__ float qh[DH];
    __shared__ float knew[DH], vnew[DH];
    __shared__ float wst[kDecWaves][2];
    __shared__ float wacc[kDecWaves][DH];
    __shared__ float wred[kDecWaves];

    const int row32 = blockIdx.x;                // b * H + h (Bs * H < 2^31)
    const int64_t row = row32;
    const int h = row32 % H;
    const int64_t b = row32 / H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane / CH, ch = lane % CH;
    const T *kring = kcache + row * (int64_t)W * DH + ch * 8;
    const T *vring = vcache + row * (int64_t)W * DH + ch * 8;
    const int nbatch = (W + SB - 1) / SB;

    // 1. The loads the setup needs go out first (the position; this head's
    //    q, k, v and memory rows; the gated form's memory-key row), then the
    //    wave's first batch of the ring, every slot inside it, valid or not:
    //    outstanding loads complete in issue order, so the setup can go on
    //    while the batch is still in flight.
    const int64_t p = pos[b];
    const int i = tid & (DH / 2 - 1);   // rotation pair of thread tid < DH/2 (the rest load the same)
    const int64_t mrow = b * mem_stride + (int64_t)h * DH;
    const T q_lo = q[row * DH + i], q_hi = q[row * DH + i + DH / 2];
    const T k_lo = k[row * DH + i], k_hi = k[row * DH + i + DH / 2];
    const T v_lo = v[row * DH + i], v_hi = v[row * DH + i + DH / 2];
    const T km_lo = km[mrow + i], km_hi = km[mrow + i + DH / 2];
    const T vm_lo = vm[mrow + i], vm_hi = vm[mrow + i + DH / 2];
    float gx[8] = {};   // gated form: this thread's first chunk of the memory-key row
    if constexpr (GATED) {
        if (tid * 8 < H * DH) load8(km + b * mem_stride + tid * 8, gx);
    }
    // kDecBuffers batch buffers in rotation: the next batches are in flight
    // while one is reduced. Every issue is unconditional (slots past the
    // ring's end re-read its last slot, and are never used), so the count of
    // loads in flight is the same on every path and no join makes a wait
    // cover the next batch.
    using Batch = Raw8<T>[2][kBatchPasses];   // [K, V][pass]
    Batch bufs[kDecBuffers];
    auto issue = [&](int j, Batch &bf) {
#pragma unroll
        for (int ps = 0; ps < kBatchPasses; ++ps) {
            int sl = j * SB + ps * G + g;
            sl = sl < W ? sl : W - 1;
            bf[0][ps].load(kring + (int64_t)sl * DH);
            bf[1][ps].load(vring + (int64_t)sl * DH);
        }
    };
#pragma unroll
    for (int u = 0; u < kDecBuffers; ++u) issue(w + u * kDecWaves, bufs[u]);
    // A stream with a negative position has no slot: it is skipped whole (ring
    // and o untouched). p is the same on every thread of the workgroup, so the
    // whole workgroup leaves before its first barrier.
    if (p < 0) return;

    // 2. Rotation of position p (double precision: no table bounds p),
    //    rotated query, and the new entry (written by this workgroup only).
    float rs = 0.0f;   // gated form: 1 / rms of the stream's memory-key row
    if constexpr (GATED) {
        const int HD = H * DH;
        const T *kpr = km + b * mem_stride;
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += gx[e] * gx[e];
        for (int c = (tid + kDecThreads) * 8; c < HD; c += kDecThreads * 8) {   // rows past 8 * kDecThreads
            float x[8];
            load8(kpr + c, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
        }
        ss = wave_sum(ss);
        if (lane == 0) wred[w] = ss;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) tot += wred[ww];
        rs = rsqrtf(tot / (float)HD + eps);
    }
    const int slot_new = (int)(p % W);
    const int nvalid = p + 1 < (int64_t)W ? (int)(p + 1) : W;   // slots 0 .. nvalid-1 hold positions >= 0
    if (tid < DH / 2) {
        float cs = 1.0f, sn = 0.0f;
        if (rope_base > 0.0f) {
            // theta_i = base^(-2i/Dh) and the angle p * theta_i in double
            // precision, reduced to [-pi, pi] in double (two-term 2*pi), then
            // the float sine and cosine of the reduced angle.
            const double theta = exp2(-(2.0 * (double)i / (double)DH) * log2_base);
            const double phi = (double)p * theta;
            const double kq = rint(phi * 0.15915494309189535);          // 1 / (2 pi)
            double r = fma(-kq, 6.283185307179586, phi);                  // 2 pi, leading part
            r = fma(-kq, 2.4492935982947064e-16, r);                      // 2 pi, remainder
            sincosf((float)r, &sn, &cs);
        }
        const float a0 = to_f<T>(q_lo), a1 = to_f<T>(q_hi);
        const float ls = scale * kLog2e;
        qh[i] = (a0 * cs - a1 * sn) * ls;
        qh[i + DH / 2] = (a0 * sn + a1 * cs) * ls;
        const float l0 = to_f<T>(k_lo), l1 = to_f<T>(k_hi);
        const float m0 = to_f<T>(km_lo), m1 = to_f<T>(km_hi);
        const float u0 = to_f<T>(v_lo), u1 = to_f<T>(v_hi);
        const float w0 = to_f<T>(vm_lo), w1 = to_f<T>(vm_hi);
        T k0, k1, v0, v1;
        if constexpr (GATED) {
            const int HD = H * DH;
            const int c0 = h * DH + i, c1 = c0 + DH / 2;
            auto g2 = [&](int which, int c) { return 2.0f * gate_sigmoid(gates[which * HD + c]); };
            const float n0 = m0 * rs, n1 = m1 * rs;
            k0 = from_f<T>(g2(0, c0) * (l0 * cs - l1 * sn) + g2(1, c0) * (n0 * cs - n1 * sn));
            k1 = from_f<T>(g2(0, c1) * (l0 * sn + l1 * cs) + g2(1, c1) * (n0 * sn + n1 * cs));
            v0 = from_f<T>(g2(2, c0) * u0 + g2(3, c0) * w0);
            v1 = from_f<T>(g2(2, c1) * u1 + g2(3, c1) * w1);
        } else {
            const float sg = gate_sigmoid(gate[h]);
            const float x0 = l0 + sg * m0, x1 = l1 + sg * m1;
            k0 = from_f<T>(x0 * cs - x1 * sn);
            k1 = from_f<T>(x0 * sn + x1 * cs);
            v0 = from_f<T>(u0 + sg * w0);
            v1 = from_f<T>(u1 + sg * w1);
        }
        knew[i] = to_f<T>(k0); knew[i + DH / 2] = to_f<T>(k1);
        vnew[i] = to_f<T>(v0); vnew[i + DH / 2] = to_f<T>(v1);
        // Whatever any wave reads from this slot (old or new contents) is
        // replaced by knew/vnew, so the write needs no ordering with the loads.
        T *kc = kcache + (row * W + slot_new) * DH;
        T *vc = vcache + (row * W + slot_new) * DH;
        kc[i] = k0; kc[i + DH / 2] = k1;
        vc[i] = v0; vc[i + DH / 2] = v1;
    }
    __syncthreads();

    float qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = qh[ch * 8 + e];

    // 3. Batches of this wave, online softmax per lane group.
    float m_run = -INFINITY, l_run = 0.0f, acc[8] = {};
    auto batch = [&](int j, const Batch &cur) {
        float sc[kBatchPasses];
        float bmax = -INFINITY;
#pragma unroll
        for (int ps = 0; ps < kBatchPasses; ++ps) {
            const int sl = j * SB + ps * G + g;
            float kv[8];
            if (sl == slot_new) {
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[e] = knew[ch * 8 + e];
            } else {
                cur[0][ps].get(kv);
            }
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d += qv[e] * kv[e];
            d = group_sum_dpp<CH>(d);
            sc[ps] = sl < nvalid ? d : -INFINITY;
            bmax = fmaxf(bmax, sc[ps]);
        }
        if (bmax == -INFINITY) return;           // nothing valid in this batch for this group
        const float mn = fmaxf(m_run, bmax);
        const float corr = m_run == -INFINITY ? 0.0f : exp2f(m_run - mn);
        l_run *= corr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= corr;
#pragma unroll
        for (int ps = 0; ps < kBatchPasses; ++ps) {
            const int sl = j * SB + ps * G + g;
            if (sl >= nvalid) continue;          // never read: an unwritten slot may hold anything
            const float pr = exp2f(sc[ps] - mn);
            float vv[8];
            if (sl == slot_new) {
#pragma unroll
                for (int e = 0; e < 8; ++e) vv[e] = vnew[ch * 8 + e];
            } else {
                cur[1][ps].get(vv);
            }
            l_run += pr;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += pr * vv[e];
        }
        m_run = mn;
    };
    // The same for a batch whose slots all hold positions >= 0 and none of
    // which is the new entry's (all batches of a full ring but one): no
    // per-slot tests. Which form a batch takes is the same on the whole wave,
    // so the choice is a scalar branch; the per-slot tests of the general
    // form made divergent branches around every slot and cost about 4 % of
    // a decode step.
    const int jnew = slot_new / SB;
    auto batch_full = [&](const Batch &cur) {
        float sc[kBatchPasses];
        float bmax = -INFINITY;
#pragma unroll
        for (int ps = 0; ps < kBatchPasses; ++ps) {
            float kv[8];
            cur[0][ps].get(kv);
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d += qv[e] * kv[e];
            sc[ps] = group_sum_dpp<CH>(d);
            bmax = fmaxf(bmax, sc[ps]);
        }
        const float mn = fmaxf(m_run, bmax);
        const float corr = m_run == -INFINITY ? 0.0f : exp2f(m_run - mn);
        l_run *= corr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= corr;
#pragma unroll
        for (int ps = 0; ps < kBatchPasses; ++ps) {
            const float pr = exp2f(sc[ps] - mn);
            float vv[8];
            cur[1][ps].get(vv);
            l_run += pr;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += pr * vv[e];
        }
        m_run = mn;
    };
    for (int j = w; j < nbatch; j += kDecBuffers * kDecWaves) {
#pragma unroll
        for (int u = 0; u < kDecBuffers; ++u) {
            const int jj = j + u * kDecWaves;
            if (jj < nbatch) {
                if (jj != jnew && (jj + 1) * SB <= nvalid) batch_full(bufs[u]);
                else batch(jj, bufs[u]);
            }
            issue(j + (u + kDecBuffers) * kDecWaves, bufs[u]);
        }
    }

    // 4. Merge the lane groups of the wave (same channels, other slots), then the waves.
#pragma unroll
    for (int off = CH; off < 64; off <<= 1) {
        const float m2 = __shfl_xor(m_run, off, 64), l2 = __shfl_xor(l_run, off, 64);
        float a2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a2[e] = __shfl_xor(acc[e], off, 64);
        merge_state<8>(m_run, l_run, acc, m2, l2, a2);
    }
    if (g == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) wacc[w][ch * 8 + e] = acc[e];
        if (ch == 0) {
            wst[w][0] = m_run;
            wst[w][1] = l_run;
        }
    }
    __syncthreads();
    if (tid < DH) {
        float m = -INFINITY, l = 0.0f, a = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) {
            const float a2 = wacc[ww][tid];
            merge_state<1>(m, l, &a, wst[ww][0], wst[ww][1], &a2);
        }
        o[row * DH + tid] = from_f<T>(a / l);
    }
}

template <typename T, int DH, bool GATED>
static void launch_decode_t(int Bs, int H, int W, float rope_base, float scale, const void *q,
                            const void *k, const void *v, const void *km, const void *vm,
                            int64_t mem_stride, const float *gate, const float *gates, float eps,
                            void *kc, void *vc, const int64_t *pos, void *o, hipStream_t s)
{
    prof::Scope ts(GATED ? "decode_step_gated" : "decode_step", s);
    hipLaunchKernelGGL((decode_kernel<T, DH, GATED>), dim3((unsigned)((int64_t)Bs * H)),
                       dim3(kDecThreads), 0, s, H, W, rope_base,
                       rope_base > 0.0f ? log2((double)rope_base) : 0.0, scale,
                       static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), static_cast<const T *>(km),
                       static_cast<const T *>(vm), mem_stride, gate, gates, eps,
                       static_cast<T *>(kc), static_cast<T *>(vc), pos, static_cast<T *>(o));
}

template <typename T, int DH>
static void launch_decode_dt(int Bs, int H, int W, float rope_base, float scale, const void *q,
                             const void *k, const void *v, const void *km, const void *vm,
                             int64_t mem_stride, const float *gate, const float *gates, float eps,
                             void *kc, void *vc, const int64_t *pos, void *o, hipStream_t s)
{
    if (gates)
        launch_decode_t<T, DH, true>(Bs, H, W, rope_base, scale, q, k, v, km, vm, mem_stride,
                                     gate, gates, eps, kc, vc, pos, o, s);
    else
        launch_decode_t<T, DH, false>(Bs, H, W, rope_base, scale, q, k, v, km, vm, mem_stride,
                                      gate, gates, eps, kc, vc, pos, o, s);
}

hipError_t launch_decode(int Bs, int H, int Dh, int W, float rope_base, float scale, int dtype,
                         const void *q, const void *k, const void *v, const void *km,
                         const void *vm, int64_t mem_stride, const float *gate,
                         const float *gates, float eps, void *kc, void *vc, const int64_t *pos,
                         void *o, void *, hipStream_t s)
{
    if (dtype == MAGLEV_BF16) {
        if (Dh == 128)
            launch_decode_dt<bf16, 128>(Bs, H, W, rope_base, scale, q, k, v, km, vm, mem_stride, gate, gates, eps, kc, vc, pos, o, s);
        else
            launch_decode_dt<bf16, 64>(Bs, H, W, rope_base, scale, q, k, v, km, vm, mem_stride, gate, gates, eps, kc, vc, pos, o, s);
    } else {
        if (Dh == 128)
            launch_decode_dt<float, 128>(Bs, H, W, rope_base, scale, q, k, v, km, vm, mem_stride, gate, gates, eps, kc, vc, pos, o, s);
        else
            launch_decode_dt<float, 64>(Bs, H, W, rope_base, scale, q, k, v, km, vm, mem_stride, gate, gates, eps, kc, vc, pos, o, s);
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
