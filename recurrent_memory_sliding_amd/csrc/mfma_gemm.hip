// mfma_gemm.hip -- bf16 MFMA GEMMs of the memory projection and its backward.
//
// Method: Maglev summary on paper.rainbus.top ("Maglev：滑动窗口循环记忆"),
// section 方法步骤详情: the recurrent K/V features are a projection of the
// shifted memory m'_{t-1} (m'_0 = 0). Forward: [kmem | vmem] = X [W_Km; W_Vm]^T
// with X row (b,t) = m'[b,t-1]. Backward (chain rule): dX = [s dk | s dv] [W_Km; W_Vm]
// lands on m'[b,t-1]; dW = s_h [dk | dv]^T X.
//
// One kernel template serves the three products. Each operand tile is staged
// in LDS in the layout it has in memory (16-byte global loads along the
// contiguous dimension). An operand whose reduction index is contiguous is
// read with ds_read_b128; one whose reduction index is the row index is read
// with the gfx950 transpose read ds_read_b64_tr_b16, so no operand is ever
// transposed in memory. Shifts and zero rows are folded into the row
// pointers; the sigma gate is folded into a pre-scaled weight copy (dX) or the
// epilogue (dW).
#include "common.hpp"
#include "mfma_kernels.hpp"

namespace maglev {
namespace mfma {

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NT = WM_ * WN_ * 64;
    static constexpr int FM = BM_ / WM_ / 32;   // 32x32 blocks per wave along M
    static constexpr int FN = BN_ / WN_ / 32;
};

// LDS footprint of one operand tile. K-major: [R][BK + 8] (row stride 80 B for
// BK = 32: conflict-free 16-byte reads). MN-major: [BK][R + 32] (row stride
// 320 B for R = 128: conflict-free transpose reads per half wave).
template <bool KMAJOR, int R, int BK>
struct OpTile {
    static constexpr int STRIDE = KMAJOR ? BK + 8 : R + 32;
    static constexpr int ROWS = KMAJOR ? R : BK;
    static constexpr int ELEMS = ROWS * STRIDE;
    static constexpr int CHUNKS = R * BK / 8;
};

MAGLEV_DEV bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

template <bool KMAJOR, int STRIDE>
MAGLEV_DEV bf16x8 read_frag(const bf16 *lds, int rb, int ks, int lane)
{
    if constexpr (KMAJOR) {
        return *reinterpret_cast<const bf16x8 *>(lds + (rb * 32 + (lane & 31)) * STRIDE + ks * 16 +
                                                 8 * (lane >> 5));
    } else {
        const int n0 = rb * 32 + 16 * ((lane >> 4) & 1);
        const int k0 = ks * 16 + 8 * (lane >> 5);
        const int j = lane & 15;
        const i16x4 lo = lds_read_tr16(lds + (k0 + (j >> 2)) * STRIDE + n0 + 4 * (j & 3));
        const i16x4 hi = lds_read_tr16(lds + (k0 + 4 + (j >> 2)) * STRIDE + n0 + 4 * (j & 3));
        return join_tr(lo, hi);
    }
}

// C[M,N] = sum_k A(m,k) B(n,k) over k in this workgroup's split.
// P supplies: M, N, K; A_KMAJOR/B_KMAJOR; a_ptr/b_ptr giving the address of
// 8 consecutive elements along the contiguous dimension (nullptr = zeros);
// store(m, n, value, split).
template <class Cfg, class P>
__global__ __launch_bounds__(Cfg::NT) void gemm_bf16(P p, int64_t kper)
{
    using TA = OpTile<P::A_KMAJOR, Cfg::BM, Cfg::BK>;
    using TB = OpTile<P::B_KMAJOR, Cfg::BN, Cfg::BK>;
    constexpr int CA = TA::CHUNKS / Cfg::NT;
    constexpr int CB = TB::CHUNKS / Cfg::NT;
    static_assert(TA::CHUNKS % Cfg::NT == 0 && TB::CHUNKS % Cfg::NT == 0, "tile/thread mismatch");
    __shared__ __attribute__((aligned(16))) bf16 lds[2][TA::ELEMS + TB::ELEMS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const int64_t ntn = (p.N + Cfg::BN - 1) / Cfg::BN;
    const int64_t ntm = (p.M + Cfg::BM - 1) / Cfg::BM;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t tm = bid / ntn, tn = bid % ntn;
    if (tm >= ntm) return;
    const int64_t m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
    const int64_t kb = (int64_t)blockIdx.z * kper;
    const int64_t ke = kb + kper < p.K ? kb + kper : p.K;
    const int nk = ke > kb ? (int)((ke - kb + Cfg::BK - 1) / Cfg::BK) : 0;

    bf16x8 ra[CA], rb[CB];
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = tid + i * Cfg::NT;
            const bf16 *src;
            if constexpr (P::A_KMAJOR) {
                const int r = c / (Cfg::BK / 8), kc = c % (Cfg::BK / 8);
                src = (k0 + 8 * kc < ke) ? p.a_ptr(m0 + r, k0 + 8 * kc) : nullptr;
            } else {
                const int kr = c / (Cfg::BM / 8), mc = c % (Cfg::BM / 8);
                src = (k0 + kr < ke) ? p.a_ptr(k0 + kr, m0 + 8 * mc) : nullptr;
            }
            ra[i] = src ? *reinterpret_cast<const bf16x8 *>(src) : zero8();
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = tid + i * Cfg::NT;
            const bf16 *src;
            if constexpr (P::B_KMAJOR) {
                const int r = c / (Cfg::BK / 8), kc = c % (Cfg::BK / 8);
                src = (k0 + 8 * kc < ke) ? p.b_ptr(n0 + r, k0 + 8 * kc) : nullptr;
            } else {
                const int kr = c / (Cfg::BN / 8), nc = c % (Cfg::BN / 8);
                src = (k0 + kr < ke) ? p.b_ptr(k0 + kr, n0 + 8 * nc) : nullptr;
            }
            rb[i] = src ? *reinterpret_cast<const bf16x8 *>(src) : zero8();
        }
    };
    auto lstore = [&](int buf) {
        bf16 *la = lds[buf];
        bf16 *lb = lds[buf] + TA::ELEMS;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = tid + i * Cfg::NT;
            int off;
            if constexpr (P::A_KMAJOR) off = (c / (Cfg::BK / 8)) * TA::STRIDE + 8 * (c % (Cfg::BK / 8));
            else off = (c / (Cfg::BM / 8)) * TA::STRIDE + 8 * (c % (Cfg::BM / 8));
            *reinterpret_cast<bf16x8 *>(la + off) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = tid + i * Cfg::NT;
            int off;
            if constexpr (P::B_KMAJOR) off = (c / (Cfg::BK / 8)) * TB::STRIDE + 8 * (c % (Cfg::BK / 8));
            else off = (c / (Cfg::BN / 8)) * TB::STRIDE + 8 * (c % (Cfg::BN / 8));
            *reinterpret_cast<bf16x8 *>(lb + off) = rb[i];
        }
    };

    f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (nk > 0) {
        gload(kb);
        lstore(0);
    }
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
        const int cur = it & 1;
        if (it + 1 < nk) gload(kb + (int64_t)(it + 1) * Cfg::BK);
        const bf16 *la = lds[cur];
        const bf16 *lb = lds[cur] + TA::ELEMS;
#pragma unroll
        for (int ks = 0; ks < Cfg::BK / 16; ++ks) {
            bf16x8 af[Cfg::FM], bfr[Cfg::FN];
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
                af[i] = read_frag<P::A_KMAJOR, TA::STRIDE>(la, wm * Cfg::FM + i, ks, lane);
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j)
                bfr[j] = read_frag<P::B_KMAJOR, TB::STRIDE>(lb, wn * Cfg::FN + j, ks, lane);
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
        if (it + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    const int g = lane >> 5;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) {
            const int64_t n = n0 + (wn * Cfg::FN + j) * 32 + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + (wm * Cfg::FM + i) * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                if (m < p.M && n < p.N) p.store(m, n, acc[i][j][e], blockIdx.z);
            }
        }
}

// ---------------------------------------------------------------------------
// Problems
// ---------------------------------------------------------------------------
// kmem | vmem [N_tok, 2HD] = X [N_tok, d] * Wcat[2HD, d]^T
struct ProjFwd {
    static constexpr bool A_KMAJOR = true, B_KMAJOR = true;
    const bf16 *m, *wk, *wv;
    bf16 *km, *vm;
    int64_t M, N, K, T;
    int HD, shift;
    MAGLEV_DEV const bf16 *a_ptr(int64_t row, int64_t k) const
    {
        if (row >= M) return nullptr;
        if (row % T < shift) return nullptr;
        return m + (row - shift) * K + k;
    }
    MAGLEV_DEV const bf16 *b_ptr(int64_t n, int64_t k) const
    {
        if (n >= N) return nullptr;
        return n < HD ? wk + n * K + k : wv + (n - HD) * K + k;
    }
    MAGLEV_DEV void store(int64_t row, int64_t n, float x, int) const
    {
        if (n < HD) km[row * HD + n] = f2bf(x);
        else vm[row * HD + (n - HD)] = f2bf(x);
    }
};

// dX [N_tok, d] = G [N_tok, 2HD] * Ws [2HD, d]; row (b,t) lands on dm'[b,t-1].
struct ProjBwdDm {
    static constexpr bool A_KMAJOR = true, B_KMAJOR = false;
    const bf16 *dk, *dv, *ws;   // ws = s_h-scaled [W_Km; W_Vm]
    float *dm;
    int64_t M, N, K, T;
    int HD;
    bool acc;
    MAGLEV_DEV const bf16 *a_ptr(int64_t row, int64_t k) const
    {
        if (row >= M) return nullptr;
        return k < HD ? dk + row * HD + k : dv + row * HD + (k - HD);
    }
    MAGLEV_DEV const bf16 *b_ptr(int64_t k, int64_t n) const
    {
        if (n >= N) return nullptr;
        return ws + k * N + n;
    }
    MAGLEV_DEV void store(int64_t row, int64_t n, float x, int) const
    {
        if (row % T == 0) return;
        float *p = dm + (row - 1) * N + n;
        *p = acc ? *p + x : x;
    }
};

// dW [2HD, d] = G^T [2HD, N_tok] * X [N_tok, d], one split of the token range.
struct ProjBwdDw {
    static constexpr bool A_KMAJOR = false, B_KMAJOR = false;
    const bf16 *dk, *dv, *m;
    float *part;      // [ksplit][2HD][d]
    int64_t M, N, K, T;
    int HD;
    MAGLEV_DEV const bf16 *a_ptr(int64_t tok, int64_t r) const
    {
        if (r >= M) return nullptr;
        return r < HD ? dk + tok * HD + r : dv + tok * HD + (r - HD);
    }
    MAGLEV_DEV const bf16 *b_ptr(int64_t tok, int64_t e) const
    {
        if (e >= N) return nullptr;
        if (tok % T == 0) return nullptr;
        return m + (tok - 1) * N + e;
    }
    MAGLEV_DEV void store(int64_t r, int64_t e, float x, int split) const
    {
        part[((int64_t)split * M + r) * N + e] = x;
    }
};

using GemmCfg = TileCfg<128, 128, 32, 2, 2>;

template <class P>
static void run_gemm(const P &p, int ksplit, int64_t kper, hipStream_t s)
{
    const int64_t ntm = (p.M + GemmCfg::BM - 1) / GemmCfg::BM;
    const int64_t ntn = (p.N + GemmCfg::BN - 1) / GemmCfg::BN;
    hipLaunchKernelGGL((gemm_bf16<GemmCfg, P>), dim3((unsigned)(ntm * ntn), 1, ksplit),
                       dim3(GemmCfg::NT), 0, s, p, kper);
}

void launch_project_bf16(const Geom &g, int shift, const void *m, const void *wk, const void *wv,
                         void *km, void *vm, hipStream_t s)
{
    ProjFwd p;
    p.m = static_cast<const bf16 *>(m);
    p.wk = static_cast<const bf16 *>(wk);
    p.wv = static_cast<const bf16 *>(wv);
    p.km = static_cast<bf16 *>(km);
    p.vm = static_cast<bf16 *>(vm);
    p.M = g.N(); p.N = 2 * (int64_t)g.HD(); p.K = g.d; p.T = g.T;
    p.HD = g.HD(); p.shift = shift;
    run_gemm(p, 1, p.K, s);
}

// s_h-scaled copy of [W_Km; W_Vm] (bf16), 8 elements per thread.
__global__ void scale_weights(const bf16 *wk, const bf16 *wv, const float *gate, bf16 *out,
                              int HD, int Dh, int d)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // chunk index
    const int64_t per = (int64_t)HD * d / 8;
    if (i >= 2 * per) return;
    const bool second = i >= per;
    const int64_t j = second ? i - per : i;
    const int r = (int)((j * 8) / d);
    const float sg = gate_sigmoid(gate[r / Dh]);
    float x[8];
    load8((second ? wv : wk) + j * 8, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= sg;
    store8(out + i * 8, x);
}

// dW = s_h * sum over splits (fixed order), optionally added to the output.
__global__ void dw_reduce(const float *part, int ksplit, int HD, int Dh, int d, const float *gate,
                          float *dwk, float *dwv, bool acc)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tot = 2 * (int64_t)HD * d;
    if (i >= tot) return;
    float x = 0.0f;
    for (int sp = 0; sp < ksplit; ++sp) x += part[sp * tot + i];
    const int64_t r = i / d;
    const int rr = (int)(r < HD ? r : r - HD);
    x *= gate_sigmoid(gate[rr / Dh]);
    float *out = (r < HD ? dwk : dwv) + (int64_t)rr * d + (i % d);
    *out = acc ? *out + x : x;
}

int dw_ksplit(const Geom &g)
{
    const int64_t tiles = ((2 * (int64_t)g.HD() + 127) / 128) * ((g.d + 127) / 128);
    int64_t ks = (1024 + tiles - 1) / tiles;            // aim for about 4 workgroups per CU
    const int64_t max_by_k = (g.N() + 1023) / 1024;      // keep >= 1024 tokens per split
    if (ks > max_by_k) ks = max_by_k;
    if (ks > 16) ks = 16;
    if (ks < 1) ks = 1;
    return (int)ks;
}

void launch_proj_bwd_bf16(const Geom &g, const void *dk, const void *dv, const void *m_prime,
                          const void *wk, const void *wv, const float *gate, float *dm_prime,
                          float *dWk, float *dWv, unsigned acc, const BwdWorkspace &ws,
                          hipStream_t s)
{
    const int HD = g.HD();
    bf16 *wsc = static_cast<bf16 *>(ws.W_scaled);
    {
        const int64_t chunks = 2 * (int64_t)HD * g.d / 8;
        hipLaunchKernelGGL(scale_weights, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                           static_cast<const bf16 *>(wk), static_cast<const bf16 *>(wv), gate, wsc,
                           HD, g.Dh, g.d);
    }
    {
        ProjBwdDm p;
        p.dk = static_cast<const bf16 *>(dk);
        p.dv = static_cast<const bf16 *>(dv);
        p.ws = wsc;
        p.dm = dm_prime;
        p.M = g.N(); p.N = g.d; p.K = 2 * (int64_t)HD; p.T = g.T;
        p.HD = HD;
        p.acc = (acc & 1u) != 0;
        run_gemm(p, 1, p.K, s);
    }
    {
        ProjBwdDw p;
        p.dk = static_cast<const bf16 *>(dk);
        p.dv = static_cast<const bf16 *>(dv);
        p.m = static_cast<const bf16 *>(m_prime);
        p.part = ws.dW_part;
        p.M = 2 * (int64_t)HD; p.N = g.d; p.K = g.N(); p.T = g.T;
        p.HD = HD;
        const int ks = ws.ksplit;
        int64_t kper = (p.K + ks - 1) / ks;
        kper = (kper + GemmCfg::BK - 1) / GemmCfg::BK * GemmCfg::BK;
        run_gemm(p, ks, kper, s);
        const int64_t tot = 2 * (int64_t)HD * g.d;
        hipLaunchKernelGGL(dw_reduce, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s,
                           ws.dW_part, ks, HD, g.Dh, g.d, gate, dWk, dWv, (acc & 2u) != 0);
    }
}

}  // namespace mfma
}  // namespace maglev
