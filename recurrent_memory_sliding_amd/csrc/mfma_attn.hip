// mfma_attn.hip -- bf16 MFMA kernels of the injected sliding-window attention:
// forward, and the backward's row-dot, key-stationary dK/dV pass and
// query-stationary dQ pass.
//
// Method: Maglev summary on paper.rainbus.top ("Maglev：滑动窗口循环记忆"),
// sections 前置知识 (each position attends to the W most recent tokens; RoPE
// rotates q and k by absolute-position angles, the injected key included,
// before mixing) and 方法步骤详情 (the gated mix of the projected shifted
// memory into the token's own K/V entry; attention over the W most recent
// mixed entries). Mixed entries: k~_j = R_j (k_j + s_h kmem_j),
// v~_j = v_j + s_h vmem_j (R is linear, so R k + s R kmem = R (k + s kmem)).
//
// Design (gfx950): 256-thread workgroups of four 64-wide waves, each wave
// owning 32 rows; v_mfma_f32_32x32x16_bf16 with fp32 accumulation. Scores are
// computed transposed (S^T = K~ Q^T) so that each lane owns one query (or key)
// column: the softmax state is per lane, the probabilities stay in registers
// and feed the next product directly (their key order is permuted to match
// the accumulator layout, and the K/V operand is read in the same order
// through ds_read_b64_tr_b16). The mixed entries k~, v~ arrive precomputed
// (the projection call writes them), so a K/V tile is a plain copy into LDS;
// key tiles wholly outside a wave's band are skipped, and only tiles that
// straddle a band edge are masked.
#include "common.hpp"
#include "mfma_kernels.hpp"
#include "profile.hpp"

namespace maglev {
namespace mfma {

struct AttnArgs {
    const bf16 *q, *kx, *vx, *km, *vm;   // kx/vx: mixed entries k~, v~
    const float2 *rope;   // [pos][Dh/2] (cos, sin) or nullptr
    int64_t B, T;
    int H, W;
    int64_t pos0;
    float scale;
};

MAGLEV_DEV int64_t act_row(const AttnArgs &a, int64_t b, int64_t t, int h)
{
    return (b * a.T + t) * a.H + h;
}

// Rotate the channel pairs (lo[e], hi[e]) = (c0 + e, c0 + e + Dh/2) by the
// table entries cs[0..7] (forward if sign = +1, inverse if -1).
MAGLEV_DEV void rotate8(float *lo, float *hi, const float2 *cs, float sign)
{
    const f32x4 *p = reinterpret_cast<const f32x4 *>(cs);
#pragma unroll
    for (int h2 = 0; h2 < 4; ++h2) {
        const f32x4 t = p[h2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = 2 * h2 + u;
            const float c = t[2 * u], sn = sign * t[2 * u + 1];
            const float x0 = lo[e], x1 = hi[e];
            lo[e] = x0 * c - x1 * sn;
            hi[e] = x0 * sn + x1 * c;
        }
    }
}

// Stage keys [j0, j0+64) of (b, h) into LDS: Ks[kk][c] = k~_{j0+kk}[c],
// Vs[kk][c] = v~_{j0+kk}[c]; rows outside [0, T) are zero.
template <int DH, int KSTR, int VSTR>
MAGLEV_DEV void stage_kv_tile(const AttnArgs &a, int64_t b, int h, int64_t j0, bf16 *Ks, bf16 *Vs,
                              int tid)
{
    constexpr int CH = DH / 8;   // 16-byte chunks per row
#pragma unroll
    for (int u = tid; u < 64 * CH; u += 256) {
        const int kk = u / CH, cc = u % CH;
        const int64_t j = j0 + kk;
        u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
        if (j >= 0 && j < a.T) {
            const int64_t base = act_row(a, b, j, h) * DH + 8 * cc;
            kv = *reinterpret_cast<const u32x4 *>(a.kx + base);
            vv = *reinterpret_cast<const u32x4 *>(a.vx + base);
        }
        *reinterpret_cast<u32x4 *>(Ks + kk * KSTR + 8 * cc) = kv;
        *reinterpret_cast<u32x4 *>(Vs + kk * VSTR + 8 * cc) = vv;
    }
}

// Per-lane operand rows of one token in the 32x32x16 layout: fragment s holds
// channels 16s + 8g .. +7 (g = lane / 32). With rotate, fragments s and
// s + DH/32 (channels c and c + DH/2) are rotated together at position t.
template <int DH>
MAGLEV_DEV void token_frags(const AttnArgs &a, const bf16 *src, int64_t t, int g, bool rotate,
                            float mul, bf16x8 *f)
{
    constexpr int HS = DH / 32;
#pragma unroll
    for (int s = 0; s < HS; ++s) {
        float lo[8], hi[8];
        const int c0 = 16 * s + 8 * g;
        load8(src + c0, lo);
        load8(src + c0 + DH / 2, hi);
        if (rotate && a.rope) rotate8(lo, hi, a.rope + (a.pos0 + t) * (DH / 2) + c0, 1.0f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo[e] *= mul;
            hi[e] *= mul;
        }
        f[s] = pack8(lo);
        f[s + HS] = pack8(hi);
    }
}

MAGLEV_DEV void zero_frags(bf16x8 *f, int n)
{
    for (int i = 0; i < n; ++i) f[i] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Transpose-read operand: rows k0..k0+3 and k0+8..k0+11 (k0 = 16 t + 4 g) of
// an LDS tile [rows][STR], columns 32 db + (lane % 32): the key/query order of
// the probabilities held in the score accumulator.
template <int STR>
MAGLEV_DEV bf16x8 tr_operand(const bf16 *lds, int t, int db, int lane)
{
    const int g = lane >> 5, j = lane & 15;
    const int n0 = 32 * db + 16 * ((lane >> 4) & 1);
    const int k0 = 16 * t + 4 * g;
    const i16x4 lo = lds_read_tr16(lds + (k0 + (j >> 2)) * STR + n0 + 4 * (j & 3));
    const i16x4 hi = lds_read_tr16(lds + (k0 + 8 + (j >> 2)) * STR + n0 + 4 * (j & 3));
    return join_tr(lo, hi);
}

// Accumulator elements 8 (t % 2) .. +7 of block t / 2 as one bf16 operand.
MAGLEV_DEV bf16x8 acc_to_operand(const f32x16 &x, int half)
{
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = f2bf(x[8 * half + e]);
    return r;
}

// ============================================================================
// Forward
// ============================================================================
template <int DH>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a, bf16 *o, float *lse)
{
    constexpr int KSTR = DH + 8;    // 16-byte reads, conflict-free per 16 lanes
    constexpr int VSTR = 160;       // transpose reads, conflict-free per half wave
    constexpr int NF = DH / 16, NB = DH / 32;
    __shared__ __attribute__((aligned(16))) bf16 Ks[64 * KSTR];
    __shared__ __attribute__((aligned(16))) bf16 Vs[64 * VSTR];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
    const int64_t nqt = (a.T + 127) / 128;
    const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t qt = bid % nqt, bh = bid / nqt;
    const int h = (int)(bh % a.H);
    const int64_t b = bh / a.H;
    const int64_t i0 = qt * 128, qw0 = i0 + 32 * w, qi = qw0 + l32;

    bf16x8 qf[NF];
    if (qi < a.T) token_frags<DH>(a, a.q + act_row(a, b, qi, h) * DH, qi, g, true, a.scale * kLog2e, qf);
    else zero_frags(qf, NF);

    f32x16 acc[NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    const int64_t klo = i0 - a.W + 1 > 0 ? i0 - a.W + 1 : 0;
    const int64_t khi = i0 + 128 < a.T ? i0 + 128 : a.T;
    const bool active = qw0 < a.T;
    const int64_t wlo = qw0 - a.W + 1;
    const int64_t whi = qw0 + 31 < a.T - 1 ? qw0 + 31 : a.T - 1;

    for (int64_t j0 = (klo / 64) * 64; j0 < khi; j0 += 64) {
        __syncthreads();
        stage_kv_tile<DH, KSTR, VSTR>(a, b, h, j0, Ks, Vs, tid);
        __syncthreads();
        if (!active || j0 > whi || j0 + 63 < wlo) continue;

        f32x16 sc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sc[kb][e] = 0.0f;
#pragma unroll
            for (int s = 0; s < NF; ++s) {
                const bf16x8 af =
                    *reinterpret_cast<const bf16x8 *>(Ks + (32 * kb + l32) * KSTR + 16 * s + 8 * g);
                sc[kb] = mfma32(af, qf[s], sc[kb]);
            }
        }
        const bool inside = (j0 + 63 <= qw0) && (j0 >= qw0 + 31 - a.W + 1) && (j0 + 63 < a.T);
        if (!inside) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t key = j0 + 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
                    if (key > qi || key < qi - a.W + 1 || key >= a.T) sc[kb][e] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][e]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float rs = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = exp2f(sc[kb][e] - m_use);
                sc[kb][e] = p;
                rs += p;
            }
        rs += xor32(rs);
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
        bf16x8 pf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) pf[t] = acc_to_operand(sc[t >> 1], t & 1);
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[db] = mfma32(tr_operand<VSTR>(Vs, t, db, lane), pf[t], acc[db]);
    }

    if (qi < a.T) {
        const float inv = 1.0f / l_run;
        bf16 *orow = o + act_row(a, b, qi, h) * DH;
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                bf16x4 v4;
#pragma unroll
                for (int u = 0; u < 4; ++u) v4[u] = f2bf(acc[db][4 * i4 + u] * inv);
                *reinterpret_cast<bf16x4 *>(orow + 32 * db + 8 * i4 + 4 * g) = v4;
            }
        if (g == 0 && lse) lse[(b * a.H + h) * a.T + qi] = (m_run + log2f(l_run)) * kLn2;
    }
}

// ============================================================================
// Backward
// ============================================================================
// D[b,h,t] = sum_c dO[b,t,h,c] O[b,t,h,c]
template <int DH>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const bf16 *o, const bf16 *dO, float *D,
                                                         int64_t rows, int H, int64_t T)
{
    constexpr int CH = DH / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / CH;   // (b*T + t)*H + h
    const int ch = (int)(gid % CH);
    float d = 0.0f;
    if (row < rows) {
        float x[8], y[8];
        load8(o + row * DH + 8 * ch, x);
        load8(dO + row * DH + 8 * ch, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) d += x[e] * y[e];
    }
#pragma unroll
    for (int off = CH / 2; off > 0; off >>= 1) d += __shfl_xor(d, off, 64);
    if (row < rows && ch == 0) {
        const int h = (int)(row % H);
        const int64_t bt = row / H;
        D[((bt / T) * H + h) * T + (bt % T)] = d;
    }
}

// Key-stationary pass: each wave owns 32 keys, the workgroup 128; query tiles
// of 32 stream through LDS. Per tile: S = Q^ K~^T, P = exp(scale S - lse),
// dP = dO V~^T, dS = P (dP - D); dV~^T += dO^T P, dK~^T += Q^^T dS.
// Epilogue: dk = scale R^T dK~, dv = dV~, and the gate partial
// <kmem, dk> + <vmem, dv> summed over the workgroup's keys.
template <int DH>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(AttnArgs a, const bf16 *dO,
                                                             const float *lse, const float *D,
                                                             bf16 *dk, bf16 *dv, float *ds_part)
{
    constexpr int QSTR = DH + 8;
    constexpr int NF = DH / 16, NB = DH / 32, CP = DH / 16;
    __shared__ __attribute__((aligned(16))) bf16 Qs[32 * QSTR];
    __shared__ __attribute__((aligned(16))) bf16 dOs[32 * QSTR];
    __shared__ float Ls[32], Ds[32];
    __shared__ float red[4];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
    const int64_t nkt = (a.T + 127) / 128;
    const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t kt = bid % nkt, bh = bid / nkt;
    const int h = (int)(bh % a.H);
    const int64_t b = bh / a.H;
    const int64_t j0 = kt * 128, kw0 = j0 + 32 * w, kj = kw0 + l32;
    const float qscale = a.scale * kLog2e;

    // This lane's key: k~ and v~ as B operands (fragment s: channels 16 s + 8 g .. +7).
    bf16x8 kf[NF], vf[NF];
    if (kj < a.T) {
        const int64_t base = act_row(a, b, kj, h) * DH;
#pragma unroll
        for (int s = 0; s < NF; ++s) {
            kf[s] = *reinterpret_cast<const bf16x8 *>(a.kx + base + 16 * s + 8 * g);
            vf[s] = *reinterpret_cast<const bf16x8 *>(a.vx + base + 16 * s + 8 * g);
        }
    } else {
        zero_frags(kf, NF);
        zero_frags(vf, NF);
    }

    f32x16 dva[NB], dka[NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dva[db][e] = dka[db][e] = 0.0f;

    const int64_t qend = j0 + 127 + a.W < a.T ? j0 + 127 + a.W : a.T;   // exclusive
    const bool active = kw0 < a.T;
    for (int64_t i0 = j0; i0 < qend; i0 += 32) {
        __syncthreads();
        // stage Q^ (rotated) and dO for queries i0 .. i0+31
        for (int u = tid; u < 32 * CP; u += 256) {
            const int qq = u / CP, cc = u % CP;
            const int64_t i = i0 + qq;
            float lo[8], hi[8], dlo[8], dhi[8];
            if (i < a.T) {
                const int64_t base = act_row(a, b, i, h) * DH + 8 * cc;
                load8(a.q + base, lo);
                load8(a.q + base + DH / 2, hi);
                if (a.rope) rotate8(lo, hi, a.rope + (a.pos0 + i) * (DH / 2) + 8 * cc, 1.0f);
                load8(dO + base, dlo);
                load8(dO + base + DH / 2, dhi);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) lo[e] = hi[e] = dlo[e] = dhi[e] = 0.0f;
            }
            store8(Qs + qq * QSTR + 8 * cc, lo);
            store8(Qs + qq * QSTR + DH / 2 + 8 * cc, hi);
            store8(dOs + qq * QSTR + 8 * cc, dlo);
            store8(dOs + qq * QSTR + DH / 2 + 8 * cc, dhi);
        }
        if (tid < 32) {
            const int64_t i = i0 + tid;
            Ls[tid] = i < a.T ? lse[(b * a.H + h) * a.T + i] * kLog2e : 0.0f;
            Ds[tid] = i < a.T ? D[(b * a.H + h) * a.T + i] : 0.0f;
        }
        __syncthreads();
        if (!active || i0 + 31 < kw0 || i0 > kw0 + 31 + a.W - 1) continue;

        f32x16 sc, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[e] = dp[e] = 0.0f;
#pragma unroll
        for (int s = 0; s < NF; ++s) {
            const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(Qs + l32 * QSTR + 16 * s + 8 * g);
            sc = mfma32(qa, kf[s], sc);
            const bf16x8 da = *reinterpret_cast<const bf16x8 *>(dOs + l32 * QSTR + 16 * s + 8 * g);
            dp = mfma32(da, vf[s], dp);
        }
        // element e: query i0 + 8(e/4) + 4g + e%4, key kj
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int qq = 8 * (e >> 2) + 4 * g + (e & 3);
            const int64_t i = i0 + qq;
            const bool ok = i >= kj && i - kj < a.W && i < a.T;
            const float p = ok ? exp2f(sc[e] * qscale - Ls[qq]) : 0.0f;
            sc[e] = p;
            dp[e] = p * (dp[e] - Ds[qq]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bf16x8 pf = acc_to_operand(sc, t);
            const bf16x8 dsf = acc_to_operand(dp, t);
#pragma unroll
            for (int db = 0; db < NB; ++db) {
                dva[db] = mfma32(tr_operand<QSTR>(dOs, t, db, lane), pf, dva[db]);
                dka[db] = mfma32(tr_operand<QSTR>(Qs, t, db, lane), dsf, dka[db]);
            }
        }
    }

    // Epilogue: element e of block db is channel 32 db + 8(e/4) + 4g + e%4 of key kj.
    float part = 0.0f;
    if (kj < a.T) {
        const int64_t base = act_row(a, b, kj, h) * DH;
        const float2 *cs = a.rope ? a.rope + (a.pos0 + kj) * (DH / 2) : nullptr;
#pragma unroll
        for (int db = 0; db < NB / 2; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int c = 32 * db + 8 * (e >> 2) + 4 * g + (e & 3);
                const float lo = dka[db][e] * a.scale, hi = dka[db + NB / 2][e] * a.scale;
                if (cs) {
                    const float2 r = cs[c];
                    dka[db][e] = lo * r.x + hi * r.y;
                    dka[db + NB / 2][e] = -lo * r.y + hi * r.x;
                } else {
                    dka[db][e] = lo;
                    dka[db + NB / 2][e] = hi;
                }
            }
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int c = 32 * db + 8 * i4 + 4 * g;
                bf16x4 k4, v4;
                const bf16x4 km4 = *reinterpret_cast<const bf16x4 *>(a.km + base + c);
                const bf16x4 vm4 = *reinterpret_cast<const bf16x4 *>(a.vm + base + c);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float dkv = dka[db][4 * i4 + u], dvv = dva[db][4 * i4 + u];
                    k4[u] = f2bf(dkv);
                    v4[u] = f2bf(dvv);
                    part += dkv * bf2f(km4[u]) + dvv * bf2f(vm4[u]);
                }
                *reinterpret_cast<bf16x4 *>(dk + base + c) = k4;
                *reinterpret_cast<bf16x4 *>(dv + base + c) = v4;
            }
    }
    part = wave_sum(part);
    if (lane == 0) red[w] = part;
    __syncthreads();
    if (tid == 0) ds_part[(b * a.H + h) * nkt + kt] = red[0] + red[1] + red[2] + red[3];
}

// Query-stationary pass: each wave owns 32 queries; key tiles of 64 in the
// band stream through LDS (mixed on load). Per tile: S^T = K~ Q^^T,
// P^T = exp(scale S^T - lse), dP^T = V~ dO^T, dS^T = P^T (dP^T - D),
// dQ^^T += K~^T dS^T. Epilogue: dq = scale R^T dQ^.
template <int DH>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(AttnArgs a, const bf16 *dO,
                                                              const float *lse, const float *D,
                                                              bf16 *dq)
{
    constexpr int KSTR = DH + 8, VSTR = DH + 8;
    constexpr int NF = DH / 16, NB = DH / 32;
    __shared__ __attribute__((aligned(16))) bf16 Ks[64 * KSTR];
    __shared__ __attribute__((aligned(16))) bf16 Vs[64 * VSTR];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
    const int64_t nqt = (a.T + 127) / 128;
    const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t qt = bid % nqt, bh = bid / nqt;
    const int h = (int)(bh % a.H);
    const int64_t b = bh / a.H;
    const int64_t i0 = qt * 128, qw0 = i0 + 32 * w, qi = qw0 + l32;

    bf16x8 qf[NF], df[NF];
    float lse2 = 0.0f, Dq = 0.0f;
    if (qi < a.T) {
        const int64_t base = act_row(a, b, qi, h) * DH;
        token_frags<DH>(a, a.q + base, qi, g, true, a.scale * kLog2e, qf);
        token_frags<DH>(a, dO + base, qi, g, false, 1.0f, df);
        lse2 = lse[(b * a.H + h) * a.T + qi] * kLog2e;
        Dq = D[(b * a.H + h) * a.T + qi];
    } else {
        zero_frags(qf, NF);
        zero_frags(df, NF);
    }
    f32x16 acc[NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;

    const int64_t klo = i0 - a.W + 1 > 0 ? i0 - a.W + 1 : 0;
    const int64_t khi = i0 + 128 < a.T ? i0 + 128 : a.T;
    const bool active = qw0 < a.T;
    const int64_t wlo = qw0 - a.W + 1;
    const int64_t whi = qw0 + 31 < a.T - 1 ? qw0 + 31 : a.T - 1;

    for (int64_t j0 = (klo / 64) * 64; j0 < khi; j0 += 64) {
        __syncthreads();
        stage_kv_tile<DH, KSTR, VSTR>(a, b, h, j0, Ks, Vs, tid);
        __syncthreads();
        if (!active || j0 > whi || j0 + 63 < wlo) continue;

        f32x16 sc[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sc[kb][e] = dp[kb][e] = 0.0f;
#pragma unroll
            for (int s = 0; s < NF; ++s) {
                const bf16x8 ka =
                    *reinterpret_cast<const bf16x8 *>(Ks + (32 * kb + l32) * KSTR + 16 * s + 8 * g);
                sc[kb] = mfma32(ka, qf[s], sc[kb]);
                const bf16x8 va =
                    *reinterpret_cast<const bf16x8 *>(Vs + (32 * kb + l32) * VSTR + 16 * s + 8 * g);
                dp[kb] = mfma32(va, df[s], dp[kb]);
            }
        }
        const bool inside = (j0 + 63 <= qw0) && (j0 >= qw0 + 31 - a.W + 1) && (j0 + 63 < a.T);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t key = j0 + 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
                const bool ok = inside || (key <= qi && key > qi - a.W && key < a.T);
                const float p = ok ? exp2f(sc[kb][e] - lse2) : 0.0f;
                dp[kb][e] = p * (dp[kb][e] - Dq);
            }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bf16x8 dsf = acc_to_operand(dp[t >> 1], t & 1);
#pragma unroll
            for (int db = 0; db < NB; ++db) acc[db] = mfma32(tr_operand<KSTR>(Ks, t, db, lane), dsf, acc[db]);
        }
    }

    if (qi < a.T) {
        const int64_t base = act_row(a, b, qi, h) * DH;
        const float2 *cs = a.rope ? a.rope + (a.pos0 + qi) * (DH / 2) : nullptr;
#pragma unroll
        for (int db = 0; db < NB / 2; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int c = 32 * db + 8 * (e >> 2) + 4 * g + (e & 3);
                const float lo = acc[db][e] * a.scale, hi = acc[db + NB / 2][e] * a.scale;
                if (cs) {
                    const float2 r = cs[c];
                    acc[db][e] = lo * r.x + hi * r.y;
                    acc[db + NB / 2][e] = -lo * r.y + hi * r.x;
                } else {
                    acc[db][e] = lo;
                    acc[db + NB / 2][e] = hi;
                }
            }
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                bf16x4 v4;
#pragma unroll
                for (int u = 0; u < 4; ++u) v4[u] = f2bf(acc[db][4 * i4 + u]);
                *reinterpret_cast<bf16x4 *>(dq + base + 32 * db + 8 * i4 + 4 * g) = v4;
            }
    }
}

// ============================================================================
// Launchers
// ============================================================================
static AttnArgs make_args(const Geom &g, const void *q, const void *kx, const void *vx,
                          const void *km, const void *vm, const float2 *rope)
{
    AttnArgs a;
    a.q = static_cast<const bf16 *>(q);
    a.kx = static_cast<const bf16 *>(kx);
    a.vx = static_cast<const bf16 *>(vx);
    a.km = static_cast<const bf16 *>(km);
    a.vm = static_cast<const bf16 *>(vm);
    a.rope = rope;
    a.B = g.B; a.T = g.T; a.H = g.H; a.W = g.W; a.pos0 = g.pos0; a.scale = g.scale;
    return a;
}

void launch_attn_fwd_bf16(const Geom &g, const void *q, const void *kx, const void *vx,
                          const float2 *rope, void *o, float *lse, hipStream_t s)
{
    const AttnArgs a = make_args(g, q, kx, vx, nullptr, nullptr, rope);
    const unsigned nwg = (unsigned)(g.B * g.H * ((g.T + 127) / 128));
    prof::Scope ts("attn_fwd", s);
    if (g.Dh == 128)
        hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(nwg), dim3(256), 0, s, a, static_cast<bf16 *>(o), lse);
    else
        hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(nwg), dim3(256), 0, s, a, static_cast<bf16 *>(o), lse);
}

int64_t ds_part_per_bh(const Geom &g) { return (g.T + 127) / 128; }

template <int DH>
static void launch_attn_bwd_t(const AttnArgs &a, const bf16 *o, const bf16 *dO, const float *lse,
                              void *dq, void *dk, void *dv, const BwdWorkspace &ws, int64_t rows,
                              unsigned pre_blocks, unsigned nwg, hipStream_t s)
{
    {
        prof::Scope ts("attn_bwd_rowdot", s);
        hipLaunchKernelGGL(bwd_rowdot_kernel<DH>, dim3(pre_blocks), dim3(256), 0, s, o, dO, ws.D,
                           rows, a.H, a.T);
    }
    {
        prof::Scope ts("attn_bwd_dkdv", s);
        hipLaunchKernelGGL(attn_bwd_dkdv_kernel<DH>, dim3(nwg), dim3(256), 0, s, a, dO, lse, ws.D,
                           static_cast<bf16 *>(dk), static_cast<bf16 *>(dv), ws.ds_part);
    }
    prof::Scope ts("attn_bwd_dq", s);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<DH>, dim3(nwg), dim3(256), 0, s, a, dO, lse, ws.D,
                       static_cast<bf16 *>(dq));
}

void launch_attn_bwd_bf16(const Geom &g, const void *q, const void *kx, const void *vx,
                          const void *km, const void *vm, const float *gate, const void *o,
                          const float *lse, const void *dO, void *dq, void *dk, void *dv,
                          const BwdWorkspace &ws, const float2 *rope, hipStream_t s)
{
    (void)gate;
    const AttnArgs a = make_args(g, q, kx, vx, km, vm, rope);
    const int64_t rows = g.N() * g.H;
    const int CH = g.Dh / 8;
    const unsigned pre_blocks = (unsigned)((rows * CH + 255) / 256);
    const unsigned nwg = (unsigned)(g.B * g.H * ((g.T + 127) / 128));
    const bf16 *ob = static_cast<const bf16 *>(o);
    const bf16 *dOb = static_cast<const bf16 *>(dO);
    if (g.Dh == 128)
        launch_attn_bwd_t<128>(a, ob, dOb, lse, dq, dk, dv, ws, rows, pre_blocks, nwg, s);
    else
        launch_attn_bwd_t<64>(a, ob, dOb, lse, dq, dk, dv, ws, rows, pre_blocks, nwg, s);
}

}  // namespace mfma
}  // namespace maglev
