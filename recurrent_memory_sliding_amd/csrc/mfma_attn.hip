// mfma_attn.hip -- bf16 MFMA kernels of the injected sliding-window attention:
// forward, and the backward's preprocess (row dot and rotated queries),
// key-stationary dK/dV pass and query-stationary dQ pass.
//
// Method: Maglev summary on paper.rainbus.top ("Maglev：滑动窗口循环记忆"),
// sections 前置知识 (each position attends to the W most recent tokens; RoPE
// rotates q and k by absolute-position angles, the injected key included,
// before mixing) and 方法步骤详情 (the gated mix of the projected shifted
// memory into the token's own K/V entry; attention over the W most recent
// mixed entries). The mixed entries k~_j = R_j (k_j + s_h kmem_j),
// v~_j = v_j + s_h vmem_j arrive precomputed (the projection call writes them).
//
// Design (gfx950): 256-thread workgroups of four 64-wide waves, each wave
// owning 32 rows; v_mfma_f32_32x32x16_bf16 with fp32 accumulation. Scores are
// computed transposed (S^T = K~ Q^T) where that makes each lane own one query
// (or key) column: the softmax state is per lane, the probabilities stay in
// registers and feed the next product directly (their key order is permuted
// to match the accumulator layout, and the other operand is read in the same
// order through ds_read_b64_tr_b16).
//
// Streamed tiles (K~/V~ in the forward and dQ passes, Q^/dO in the dK/dV pass)
// go from global memory straight into LDS (global_load_lds, 16 bytes a lane)
// through a ring of pipeline stages: the next tiles' loads are in flight
// while the current one is used. Tiles are unpadded [rows][Dh] with 16-byte chunks XOR-swizzled so
// that both the row reads (ds_read_b128, 16 rows a pass) and the transposed
// reads (4 rows x 64 bytes a half-wave pass) hit every LDS bank once. Key
// tiles wholly outside a wave's band are skipped, and only tiles that
// straddle a band edge are masked.
#include "common.hpp"
#include "mfma_kernels.hpp"
#include "profile.hpp"

namespace maglev {
namespace mfma {

struct AttnArgs {
    const bf16 *q;      // queries before rotation (forward)
    const bf16 *qr;     // rotated queries R q (backward)
    const bf16 *kx, *vx;
    const float2 *rope; // [pos][Dh/2] (cos, sin) or nullptr
    int64_t B, T;
    int H, W;
    int64_t pos0;
    float scale;
};

MAGLEV_DEV int64_t act_row(const AttnArgs &a, int64_t b, int64_t t, int h)
{
    return (b * a.T + t) * a.H + h;
}

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x2, kSchedMfma = 0x8, kSchedDsRead = 0x100;

// Source of tile rows outside the sequence.
__device__ __attribute__((aligned(256))) bf16 g_attn_zero[128] = {};

// ---------------------------------------------------------------------------
// Swizzled tiles: chunk c (8 channels) of row r sits in slot c ^ swz(r).
//   Dh = 128 (16 chunks a row, 256 bytes = all 64 banks): swz is a bijection
//     of r mod 16 (row reads: 16 rows of one chunk -> 16 slots) whose bits
//     2-3 are r mod 4 (transposed reads: 4 rows of one 64-byte group -> 4 groups).
//   Dh = 64 (8 chunks, 128 bytes: rows alternate bank halves): bijective on
//     r/2 mod 8 for the row reads; rows r, r+2 of a group differ by 64 bytes.
// ---------------------------------------------------------------------------
template <int DH>
MAGLEV_DEV int swz(int r)
{
    if constexpr (DH == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int DH>
MAGLEV_DEV int tile_off(int r, int c)
{
    return r * DH + ((c ^ swz<DH>(r)) << 3);
}

// Row operand: rows 32 rb + (lane % 32), channels 16 s + 8 (lane / 32) .. +7.
template <int DH>
MAGLEV_DEV bf16x8 tile_rows(const bf16 *t, int rb, int s, int lane)
{
    const int r = rb * 32 + (lane & 31);
    return *reinterpret_cast<const bf16x8 *>(t + tile_off<DH>(r, 2 * s + (lane >> 5)));
}

// Transposed operand: reduction rows 16 tt + 4 g + {0..3} and 16 tt + 8 + 4 g + {0..3}
// (g = lane / 32), column 32 db + (lane % 32): the row order of the
// probabilities held in a score accumulator.
template <int DH>
MAGLEV_DEV bf16x8 tile_tr(const bf16 *t, int tt, int db, int lane)
{
    const int g = lane >> 5, j = lane & 15;
    const int n = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
    const int c = n >> 3, e = n & 7;
    const int ra = 16 * tt + 4 * g + (j >> 2);
    const i16x4 lo = lds_read_tr16(t + tile_off<DH>(ra, c) + e);
    const i16x4 hi = lds_read_tr16(t + tile_off<DH>(ra + 8, c) + e);
    return join_tr(lo, hi);
}

// DMA of a ROWS x DH tile by NW waves: one instruction moves 1 KB = RPI rows.
template <int DH, int ROWS, int NW>
struct TileDma {
    static constexpr int CPR = DH / 8;
    static constexpr int RPI = 64 / CPR;
    static constexpr int INSTR = ROWS / RPI;
    static constexpr int PER_WAVE = INSTR / NW;
    static_assert(INSTR % NW == 0, "tile / wave mismatch");
    // Tile row and source chunk of this lane in instruction `ins`.
    MAGLEV_DEV static int row(int ins, int lane) { return ins * RPI + lane / CPR; }
    MAGLEV_DEV static int chunk(int r, int lane) { return (lane % CPR) ^ swz<DH>(r); }
};

// ---------------------------------------------------------------------------
// Register helpers
// ---------------------------------------------------------------------------
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

// 2^x by the hardware instruction (v_exp_f32; -inf -> 0). Its inputs here are
// scaled scores minus a row maximum or log-sum-exp (never large and positive),
// so the range fix-ups of exp2f are not needed.
MAGLEV_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

MAGLEV_DEV void zero_frags(bf16x8 *f, int n)
{
    for (int i = 0; i < n; ++i) f[i] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Accumulator elements 8 (t % 2) .. +7 of block t / 2 as one bf16 operand.
MAGLEV_DEV bf16x8 acc_to_operand(const f32x16 &x, int half)
{
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = f2bf(x[8 * half + e]);
    return r;
}

// Keys j0 .. j0+KT-1 of (b, h) from kx and vx into one K tile and one V tile
// (this wave's share); rows at or beyond T read zeros.
template <int DH, int KT>
MAGLEV_DEV void issue_kv_tile(const bf16 *kbase, const bf16 *vbase, int tok_stride, int T, int j0,
                              bf16 *kt, bf16 *vt, int w, int lane)
{
    using Dma = TileDma<DH, KT, 4>;
#pragma unroll
    for (int i = 0; i < Dma::PER_WAVE; ++i) {
        const int ins = w * Dma::PER_WAVE + i;
        const int r = Dma::row(ins, lane);
        const int c = Dma::chunk(r, lane);
        const int j = j0 + r;
        const bool in = j < T;
        const int64_t off = (int64_t)j * tok_stride + c * 8;
        dma16(in ? kbase + off : g_attn_zero, kt + ins * 512);
        dma16(in ? vbase + off : g_attn_zero, vt + ins * 512);
    }
}

// Pipeline bookkeeping shared by the streamed loops: tile `it` of nt lives in
// stage it % ST; ST - 1 tiles are issued ahead. At the top of iteration it a
// wave waits until only the (at most ST - 2) later tiles' loads of its own are
// outstanding, then the barrier makes every wave's share visible and frees
// the stage the next issue overwrites (read last in iteration it - 1).
template <int ST, int PER>
MAGLEV_DEV void pipeline_wait(int it, int nt)
{
    if (ST > 2 && it + ST - 2 < nt) wait_vmcnt<(ST > 2 ? (ST - 2) * PER : 0)>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
}

// ============================================================================
// Forward
// ============================================================================
// KT keys per tile (32 or 64), ST pipeline stages.
template <int DH, int KT, int ST>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a, bf16 *o, float *lse)
{
    constexpr int NF = DH / 16, NB = DH / 32, KB = KT / 32;
    constexpr int TE = KT * DH;                          // elements of one tile
    constexpr int PER = 2 * TileDma<DH, KT, 4>::PER_WAVE;
    __shared__ __attribute__((aligned(1024))) bf16 lds[ST * 2 * TE];   // [stage][K, V]

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = (int)a.T, W = a.W;
    const int nqt = (T + 127) / 128;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = bid % nqt, bh = bid / nqt;
    const int h = bh % a.H;
    const int64_t b = bh / a.H;
    const int i0 = qt * 128, qw0 = i0 + 32 * w, qi = qw0 + l32;
    const int tok_stride = a.H * DH;
    const bf16 *kbase = a.kx + act_row(a, b, 0, h) * DH;
    const bf16 *vbase = a.vx + act_row(a, b, 0, h) * DH;

    const int klo = i0 - W + 1 > 0 ? i0 - W + 1 : 0;
    const int khi = i0 + 128 < T ? i0 + 128 : T;
    const int jstart = (klo / KT) * KT;
    const int nt = (khi - jstart + KT - 1) / KT;
    // The query operands are complete before any tile load is issued (see the
    // dQ pass for why).
    bf16x8 qf[NF];
    if (qi < T) token_frags<DH>(a, a.q + act_row(a, b, qi, h) * DH, qi, g, true, a.scale * kLog2e, qf);
    else zero_frags(qf, NF);
    wait_vmcnt<0>();

    auto issue = [&](int it) {
        bf16 *kt = lds + (it % ST) * 2 * TE;
        issue_kv_tile<DH, KT>(kbase, vbase, tok_stride, T, jstart + it * KT, kt, kt + TE, w, lane);
    };
#pragma unroll
    for (int s0 = 0; s0 < ST - 1; ++s0)
        if (s0 < nt) issue(s0);

    f32x16 acc[NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    const bool active = qw0 < T;
    const int wlo = qw0 - W + 1;
    const int whi = qw0 + 31 < T - 1 ? qw0 + 31 : T - 1;

    for (int it = 0; it < nt; ++it) {
        pipeline_wait<ST, PER>(it, nt);
        if (it + ST - 1 < nt) issue(it + ST - 1);
        const int j0 = jstart + it * KT;
        if (!active || j0 > whi || j0 + KT - 1 < wlo) continue;
        const bf16 *kt = lds + (it % ST) * 2 * TE, *vt = kt + TE;

        f32x16 sc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            bf16x8 kf[NF];   // every LDS read of the block issued before the products
#pragma unroll
            for (int s = 0; s < NF; ++s) kf[s] = tile_rows<DH>(kt, kb, s, lane);
#pragma unroll
            for (int e = 0; e < 16; ++e) sc[kb][e] = 0.0f;
#pragma unroll
            for (int s = 0; s < NF; ++s) sc[kb] = mfma32(kf[s], qf[s], sc[kb]);
        }
        const bool inside = (j0 + KT - 1 <= qw0) && (j0 >= qw0 + 31 - W + 1) && (j0 + KT - 1 < T);
        if (!inside) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = j0 + 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
                    if ((key > qi) | (key < qi - W + 1) | (key >= T)) sc[kb][e] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][e]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float rs = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = fast_exp2(sc[kb][e] - m_use);
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
        bf16x8 pf[2 * KB], vfr[NB][2 * KB];
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int t = 0; t < 2 * KB; ++t) vfr[db][t] = tile_tr<DH>(vt, t, db, lane);
#pragma unroll
        for (int t = 0; t < 2 * KB; ++t) pf[t] = acc_to_operand(sc[t >> 1], t & 1);
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int t = 0; t < 2 * KB; ++t) acc[db] = mfma32(vfr[db][t], pf[t], acc[db]);
    }

    if (qi < T) {
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
// Preprocess, one thread per chunk pair (channels 8cc .. +7 and the same + Dh/2)
// of a (b, t, h) row:
//   Dp[b,h,t] = sum_c dO[b,t,h,c] O[b,t,h,c], lse2[b,h,t] = lse[b,h,t] log2(e)
//   (both rows padded with zeros from T to Tp), and the rotated queries qr = R_t q.
template <int DH>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const bf16 *o, const bf16 *dO, const bf16 *q,
                                                       const float *lse, const float2 *rope,
                                                       bf16 *qr, float *Dp, float *lse2,
                                                       int64_t rows, int H, int64_t T, int64_t Tp,
                                                       int64_t pos0)
{
    constexpr int CP = DH / 16;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / CP;   // (b*T + t)*H + h
    const int cc = (int)(gid % CP);
    float d = 0.0f;
    if (row < rows) {
        const int64_t base = row * DH + 8 * cc;
        float x[8], y[8];
        load8(o + base, x);
        load8(dO + base, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) d += x[e] * y[e];
        load8(o + base + DH / 2, x);
        load8(dO + base + DH / 2, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) d += x[e] * y[e];
        float lo[8], hi[8];
        load8(q + base, lo);
        load8(q + base + DH / 2, hi);
        if (rope) {
            const int64_t t = (row / H) % T;
            rotate8(lo, hi, rope + (pos0 + t) * (DH / 2) + 8 * cc, 1.0f);
        }
        store8(qr + base, lo);
        store8(qr + base + DH / 2, hi);
    }
#pragma unroll
    for (int off = CP / 2; off > 0; off >>= 1) d += __shfl_xor(d, off, 64);
    if (row < rows && cc == 0) {
        const int h = (int)(row % H);
        const int64_t bt = row / H;
        const int64_t t = bt % T;
        const int64_t bh = (bt / T) * H + h;
        Dp[bh * Tp + t] = d;
        lse2[bh * Tp + t] = lse[bh * T + t] * kLog2e;
        if (t == T - 1)
            for (int64_t u = T; u < Tp; ++u) Dp[bh * Tp + u] = lse2[bh * Tp + u] = 0.0f;
    }
}

// acc[db][e] holds channel 32 db + 8(e/4) + 4g + e%4 of one row (g = lane/32);
// channels c and c + DH/2 (blocks db and db + NB/2) form a rotation pair.
// Scales by `scale` and applies R^T of the row's table cs (nullptr: no
// rotation). The branch on cs is taken once and the table is read with
// 16-byte loads issued together (a per-element branch would make each load
// wait on its own).
template <int NB>
MAGLEV_DEV void scale_rotate_back(f32x16 *acc, const float2 *cs, int g, float scale)
{
    if (cs) {
#pragma unroll
        for (int db = 0; db < NB / 2; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float *t = reinterpret_cast<const float *>(cs + 32 * db + 8 * q + 4 * g);
                const f32x4 t0 = *reinterpret_cast<const f32x4 *>(t);
                const f32x4 t1 = *reinterpret_cast<const f32x4 *>(t + 4);
                const float cx[4] = {t0[0], t0[2], t1[0], t1[2]};
                const float sy[4] = {t0[1], t0[3], t1[1], t1[3]};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e = 4 * q + u;
                    const float lo = acc[db][e] * scale, hi = acc[db + NB / 2][e] * scale;
                    acc[db][e] = lo * cx[u] + hi * sy[u];
                    acc[db + NB / 2][e] = -lo * sy[u] + hi * cx[u];
                }
            }
    } else {
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[db][e] *= scale;
    }
}

// Key-stationary pass: each wave owns 32 keys, the workgroup 128; query tiles
// of 32 (rotated queries Q^ and dO, with their lse and D) stream through LDS.
// Per tile: S = Q^ K~^T, P = exp(scale S - lse), dP = dO V~^T,
// dS = P (dP - D); dV~^T += dO^T P, dK~^T += Q^^T dS.
// Epilogue: dk = scale R^T dK~ and dv = dV~ (with ROTATE false: scale dK~ in
// the rotated frame and dV~, the gradients of the mixed entries themselves,
// which the gated mixing form takes through its own gates, rotation and norm).
// The gate gradient of the sigma-gated form does not need this kernel: it is
// sum_t <kmem_t, dk_t> + <vmem_t, dv_t> = <W_Km, G_k> + <W_Vm, G_v> with
// G = sum_t [dk_t | dv_t] x_t^T, the product the dW GEMM computes anyway.
template <int DH, int ST, bool ROTATE>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(AttnArgs a, const bf16 *dO,
                                                             const float *lse2, const float *Dp,
                                                             int64_t Tp, bf16 *dk, bf16 *dv)
{
    constexpr int NF = DH / 16, NB = DH / 32;
    constexpr int QT = 32;
    constexpr int TE = QT * DH;
    using Dma = TileDma<DH, QT, 4>;
    constexpr int PER = 2 * Dma::PER_WAVE + 1;
    __shared__ __attribute__((aligned(1024))) bf16 lds[ST * 2 * TE];   // [stage][Q^, dO]
    __shared__ __attribute__((aligned(16))) float LD[ST][2 * QT];      // [stage][lse2, D]

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = (int)a.T, W = a.W;
    const int nkt = (T + 127) / 128;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = bid % nkt, bh = bid / nkt;
    const int h = bh % a.H;
    const int64_t b = bh / a.H;
    const int j0 = kt * 128, kw0 = j0 + 32 * w, kj = kw0 + l32;
    const float qscale = a.scale * kLog2e;
    const int tok_stride = a.H * DH;
    const bf16 *qbase = a.qr + act_row(a, b, 0, h) * DH;
    const bf16 *obase = dO + act_row(a, b, 0, h) * DH;
    const float *lrow = lse2 + (int64_t)bh * Tp;
    const float *drow = Dp + (int64_t)bh * Tp;

    const int qend = j0 + 127 + W < T ? j0 + 127 + W : T;   // exclusive
    const int nt = (qend - j0 + QT - 1) / QT;

    // This lane's key: k~ and v~ as B operands (fragment s: channels 16 s + 8 g .. +7),
    // loaded and waited for before any tile load is issued: the loop must see
    // them as complete, or the compiler waits for every load in flight (the
    // tile loads included) at their first use inside the loop.
    bf16x8 kf[NF], vf[NF];
    if (kj < T) {
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
    wait_vmcnt<0>();

    auto issue = [&](int it) {
        const int buf = it % ST;
        const int i0 = j0 + it * QT;
        bf16 *qt = lds + buf * 2 * TE, *ot = qt + TE;
#pragma unroll
        for (int i = 0; i < Dma::PER_WAVE; ++i) {
            const int ins = w * Dma::PER_WAVE + i;
            const int r = Dma::row(ins, lane);
            const int c = Dma::chunk(r, lane);
            const int qi = i0 + r;
            const bool in = qi < T;
            const int64_t off = (int64_t)qi * tok_stride + c * 8;
            dma16(in ? qbase + off : g_attn_zero, qt + ins * 512);
            dma16(in ? obase + off : g_attn_zero, ot + ins * 512);
        }
        // lse2 and D of the tile: 16 chunks of 16 bytes, four per wave (rows
        // are padded to Tp, so the tile never leaves its row).
        if (lane < 4) {
            const int q = 4 * w + lane;
            const float *src = q < 8 ? lrow + i0 + 4 * q : drow + i0 + 4 * (q - 8);
            dma16(reinterpret_cast<const bf16 *>(src), reinterpret_cast<bf16 *>(&LD[buf][16 * w]));
        }
    };
#pragma unroll
    for (int s0 = 0; s0 < ST - 1; ++s0)
        if (s0 < nt) issue(s0);

    f32x16 dva[NB], dka[NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dva[db][e] = dka[db][e] = 0.0f;

    const bool active = kw0 < T;
    for (int it = 0; it < nt; ++it) {
        pipeline_wait<ST, PER>(it, nt);
        if (it + ST - 1 < nt) issue(it + ST - 1);
        // Tiles outside this wave's band are not skipped: the mask zeroes them.
        // A skip path would make the loop-carried dK/dV accumulators merge two
        // definitions, and the compiler then keeps them in VGPRs and copies all
        // 128 into accumulation registers on every tile.
        const int i0 = j0 + it * QT;
        (void)active;
        const int buf = it % ST;
        const bf16 *qt = lds + buf * 2 * TE, *ot = qt + TE;
        const float *Ls = LD[buf], *Ds = LD[buf] + QT;

        f32x16 sc, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[e] = dp[e] = 0.0f;
#pragma unroll
        for (int s = 0; s < NF; ++s) {
            sc = mfma32(tile_rows<DH>(qt, 0, s, lane), kf[s], sc);
            dp = mfma32(tile_rows<DH>(ot, 0, s, lane), vf[s], dp);
        }
        // element e: query i0 + 8(e/4) + 4g + e%4, key kj. The lse/D values of
        // this lane's 16 queries are four 16-byte LDS reads each, read
        // unconditionally (no per-element branch around an LDS load).
        f32x4 lv[4], dv4[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            lv[q4] = *reinterpret_cast<const f32x4 *>(Ls + 8 * q4 + 4 * g);
            dv4[q4] = *reinterpret_cast<const f32x4 *>(Ds + 8 * q4 + 4 * g);
        }
        // A tile whose every (query, key) pair of this wave lies in the band
        // (the usual case) takes the branch without the per-element mask; the
        // condition is uniform over the wave.
        const bool interior = (i0 >= kw0 + 31) & (i0 + QT - 1 - kw0 < W) & (i0 + QT - 1 < T);
        if (interior) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                sc[e] = fast_exp2(sc[e] * qscale - lv[e >> 2][e & 3]);
                dp[e] = sc[e] * (dp[e] - dv4[e >> 2][e & 3]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = i0 + 8 * (e >> 2) + 4 * g + (e & 3);
                const bool ok = (i >= kj) & (i - kj < W) & (i < T);
                const float p = fast_exp2(sc[e] * qscale - lv[e >> 2][e & 3]);
                sc[e] = ok ? p : 0.0f;
                dp[e] = sc[e] * (dp[e] - dv4[e >> 2][e & 3]);
            }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bf16x8 pf = acc_to_operand(sc, t);
            const bf16x8 dsf = acc_to_operand(dp, t);
#pragma unroll
            for (int db = 0; db < NB; ++db) {
                dva[db] = mfma32(tile_tr<DH>(ot, t, db, lane), pf, dva[db]);
                dka[db] = mfma32(tile_tr<DH>(qt, t, db, lane), dsf, dka[db]);
            }
        }
    }

    // Epilogue: element e of block db is channel 32 db + 8(e/4) + 4g + e%4 of key kj.
    if (kj < T) {
        const int64_t base = act_row(a, b, kj, h) * DH;
        const float2 *cs = (a.rope && ROTATE) ? a.rope + (a.pos0 + kj) * (DH / 2) : nullptr;
        scale_rotate_back<NB>(dka, cs, g, a.scale);
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int c = 32 * db + 8 * i4 + 4 * g;
                bf16x4 k4, v4;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    k4[u] = f2bf(dka[db][4 * i4 + u]);
                    v4[u] = f2bf(dva[db][4 * i4 + u]);
                }
                *reinterpret_cast<bf16x4 *>(dk + base + c) = k4;
                *reinterpret_cast<bf16x4 *>(dv + base + c) = v4;
            }
    }
}

// Scale and inverse rotation of one channel-pair block: lo holds channels
// c = c0 + 8(e/4) + 4g + e%4 of one key, hi the channels c + DH/2; cs is the
// key's rotation table at entry c0 (nullptr: scale only).
MAGLEV_DEV void scale_rotate_pair(f32x16 &lo, f32x16 &hi, const float2 *cs, int g, float scale)
{
    if (cs) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float *t = reinterpret_cast<const float *>(cs + 8 * q + 4 * g);
            const f32x4 t0 = *reinterpret_cast<const f32x4 *>(t);
            const f32x4 t1 = *reinterpret_cast<const f32x4 *>(t + 4);
            const float cx[4] = {t0[0], t0[2], t1[0], t1[2]};
            const float sy[4] = {t0[1], t0[3], t1[1], t1[3]};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = 4 * q + u;
                const float x = lo[e] * scale, y = hi[e] * scale;
                lo[e] = x * cx[u] + y * sy[u];
                hi[e] = -x * sy[u] + y * cx[u];
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            lo[e] *= scale;
            hi[e] *= scale;
        }
    }
}

// Key-stationary pass with each 32-key block split over a pair of waves
// (Dh = 128): four waves, two pairs, 64 keys a workgroup; 32-query tiles of
// Q^ and dO stream through LDS in ST stages. Per tile, the pair's first wave
// forms S = Q^ K~^T and P = exp(scale S - lse), its second wave
// dP - D = dO V~^T - D; they swap P and dP - D through LDS (one barrier a
// tile, which also publishes the next tile's stage), both form
// dS = P (dP - D), and each
// accumulates dV~^T += dO^T P and dK~^T += Q^^T dS for its half of the
// channels: blocks hf and hf + 2 of 32 channels (hf = the wave's place in
// the pair), so that the rotation pairs (c, c + 64) stay in one wave. A wave
// holds one of K~, V~ and a quarter of the accumulators, and a workgroup
// needs 80 KB of LDS, so two workgroups share a CU: they run out of step, and
// one's MFMA work covers the other's softmax, exchange and barrier. Each
// phase issues all of its LDS operand reads before its first product (one
// read in flight per product left every product waiting for LDS latency).
// The lse (first wave) or D (second wave) values of the next tile are loaded
// into registers while the current one is used (issued before the DMA that
// follows them, so the in-order count of vector memory operations tells when
// they have arrived).
template <int ST, bool ROTATE>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_pair_kernel(AttnArgs a, const bf16 *dO,
                                                                     const float *lse2,
                                                                     const float *Dp, int64_t Tp,
                                                                     bf16 *dk, bf16 *dv)
{
    static_assert(ST >= 3, "the next tile is published one tile ahead");
    constexpr int DH = 128, NF = DH / 16, NPAIR = 2, KB = 32 * NPAIR;
    constexpr int QT = 32;
    constexpr int TE = QT * DH;
    using Dma = TileDma<DH, QT, 2 * NPAIR>;
    constexpr int PER = 2 * Dma::PER_WAVE;
    __shared__ __attribute__((aligned(1024))) bf16 lds[ST * 2 * TE];   // [stage][Q^, dO]
    // [tile parity][pair][role][quad][lane]: P (role 0) and dP - D (role 1) in
    // the accumulator layout, four 16-byte groups a lane
    __shared__ __attribute__((aligned(16))) f32x4 X[2][NPAIR][2][4][64];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pr = w >> 1, hf = w & 1;
    const int T = (int)a.T, W = a.W;
    const int nkt = (T + KB - 1) / KB;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = bid % nkt, bh = bid / nkt;
    const int h = bh % a.H;
    const int64_t b = bh / a.H;
    const int j0 = kt * KB, kw0 = j0 + 32 * pr, kj = kw0 + l32;
    const float qscale = a.scale * kLog2e;
    const int tok_stride = a.H * DH;
    const bf16 *qbase = a.qr + act_row(a, b, 0, h) * DH;
    const bf16 *obase = dO + act_row(a, b, 0, h) * DH;
    const float *lrow = lse2 + (int64_t)bh * Tp;
    const float *drow = Dp + (int64_t)bh * Tp;

    const int qend = j0 + KB - 1 + W < T ? j0 + KB - 1 + W : T;   // exclusive
    const int nt = (qend - j0 + QT - 1) / QT;

    // This lane's key row of K~ (first wave) or V~ (second wave) as B
    // operands, complete before any tile load is issued.
    bf16x8 kvf[NF];
    if (kj < T) {
        const bf16 *src = (hf ? a.vx : a.kx) + act_row(a, b, kj, h) * DH;
#pragma unroll
        for (int s = 0; s < NF; ++s) kvf[s] = *reinterpret_cast<const bf16x8 *>(src + 16 * s + 8 * g);
    } else {
        zero_frags(kvf, NF);
    }
    wait_vmcnt<0>();

    auto issue = [&](int it) {
        const int buf = it % ST;
        const int i0 = j0 + it * QT;
        bf16 *qt = lds + buf * 2 * TE, *ot = qt + TE;
#pragma unroll
        for (int i = 0; i < Dma::PER_WAVE; ++i) {
            const int ins = w * Dma::PER_WAVE + i;
            const int r = Dma::row(ins, lane);
            const int c = Dma::chunk(r, lane);
            const int qi = i0 + r;
            const bool in = qi < T;
            const int64_t off = (int64_t)qi * tok_stride + c * 8;
            dma16(in ? qbase + off : g_attn_zero, qt + ins * 512);
            dma16(in ? obase + off : g_attn_zero, ot + ins * 512);
        }
    };
    // The statistic of this lane's 16 queries of tile it that the wave's role
    // needs: lse2 (first wave, for P) or D (second wave, which sends dP - D).
    // Rows are padded to Tp, so a tile never leaves its row. Two register
    // sets, one per tile parity, so that no copy (and no wait for the loads
    // behind them) is needed.
    struct Stats {
        f32x4 v[4];
    };
    const float *srow = hf ? drow : lrow;
    auto load_stats = [&](int it, Stats &st) {
        const int i0 = j0 + it * QT;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            st.v[q4] = *reinterpret_cast<const f32x4 *>(srow + i0 + 8 * q4 + 4 * g);
    };
    Stats sa, sb;
    // Tiles 0 .. ST-2 and the statistics of tile 0 in flight; all landed and
    // tile 0 visible to every wave.
#pragma unroll
    for (int s0 = 0; s0 < ST - 1; ++s0)
        if (s0 < nt) issue(s0);
    load_stats(0, sa);
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();

    f32x16 dva[2], dka[2];   // blocks hf and hf + 2 of 32 channels
#pragma unroll
    for (int lb = 0; lb < 2; ++lb)
#pragma unroll
        for (int e = 0; e < 16; ++e) dva[lb][e] = dka[lb][e] = 0.0f;

    auto tile_step = [&](int it, const Stats &cur, Stats &next) {
        const int i0 = j0 + it * QT;
        const int buf = it % ST;
        const bf16 *qt = lds + buf * 2 * TE, *ot = qt + TE;

        // S (first wave) or dP (second wave); element e: query
        // i0 + 8(e/4) + 4g + e%4, key kj
        const bf16 *rt = hf ? ot : qt;
        f32x16 mine;
#pragma unroll
        for (int e = 0; e < 16; ++e) mine[e] = 0.0f;
        bf16x8 rows[NF];
#pragma unroll
        for (int s = 0; s < NF; ++s) rows[s] = tile_rows<DH>(rt, 0, s, lane);
#pragma unroll
        for (int s = 0; s < NF; ++s) mine = mfma32(rows[s], kvf[s], mine);
        // all eight operand reads are issued before the first product waits
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NF, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, NF, 0);
        // this tile's statistics: loaded before the last DMA issued
        if (it + ST - 2 < nt) wait_vmcnt<PER>();
        else wait_vmcnt<0>();
        if (hf == 0) {
            // every (query, key) pair of this block in the band: no mask
            const bool interior = (i0 >= kw0 + 31) & (i0 + QT - 1 - kw0 < W) & (i0 + QT - 1 < T);
            if (interior) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    mine[e] = fast_exp2(mine[e] * qscale - cur.v[e >> 2][e & 3]);
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int i = i0 + 8 * (e >> 2) + 4 * g + (e & 3);
                    const bool ok = (i >= kj) & (i - kj < W) & (i < T);
                    const float p = fast_exp2(mine[e] * qscale - cur.v[e >> 2][e & 3]);
                    mine[e] = ok ? p : 0.0f;
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) mine[e] -= cur.v[e >> 2][e & 3];
        }
        const int par = it & 1;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            X[par][pr][hf][q4][lane] = f32x4{mine[4 * q4], mine[4 * q4 + 1], mine[4 * q4 + 2], mine[4 * q4 + 3]};
        // the next tile's stage (issued one iteration ago) lands before the
        // barrier publishes it
        wait_vmcnt<0>();
        __syncthreads();
        if (it + 1 < nt) load_stats(it + 1, next);
        if (it + ST - 1 < nt) issue(it + ST - 1);   // into the stage tile it - 1 used

        // the transposed operands of this tile's eight products, read before
        // the exchange so that their latency overlaps the dS arithmetic
        bf16x8 trv[2][2], trq[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int lb = 0; lb < 2; ++lb) {
                trv[t][lb] = tile_tr<DH>(ot, t, hf + 2 * lb, lane);
                trq[t][lb] = tile_tr<DH>(qt, t, hf + 2 * lb, lane);
            }
        f32x16 P, dS;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 o = X[par][pr][hf ^ 1][q4][lane];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = 4 * q4 + u;
                P[e] = hf ? o[u] : mine[e];
                dS[e] = P[e] * (hf ? mine[e] : o[u]);   // P (dP - D)
            }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bf16x8 pf = acc_to_operand(P, t);
            const bf16x8 dsf = acc_to_operand(dS, t);
#pragma unroll
            for (int lb = 0; lb < 2; ++lb) {
                dva[lb] = mfma32(trv[t][lb], pf, dva[lb]);
                dka[lb] = mfma32(trq[t][lb], dsf, dka[lb]);
            }
        }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 20, 1);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 64, 1);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 1);
    };
    for (int it = 0; it < nt; it += 2) {
        tile_step(it, sa, sb);
        if (it + 1 < nt) tile_step(it + 1, sb, sa);
    }

    // Epilogue: element e of local block lb is channel 32 (hf + 2 lb) +
    // 8(e/4) + 4g + e%4 of key kj.
    if (kj < T) {
        const int64_t base = act_row(a, b, kj, h) * DH;
        const float2 *cs =
            (a.rope && ROTATE) ? a.rope + (a.pos0 + kj) * (DH / 2) + 32 * hf : nullptr;
        scale_rotate_pair(dka[0], dka[1], cs, g, a.scale);
#pragma unroll
        for (int lb = 0; lb < 2; ++lb)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int c = 32 * (hf + 2 * lb) + 8 * i4 + 4 * g;
                bf16x4 k4, v4;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    k4[u] = f2bf(dka[lb][4 * i4 + u]);
                    v4[u] = f2bf(dva[lb][4 * i4 + u]);
                }
                *reinterpret_cast<bf16x4 *>(dk + base + c) = k4;
                *reinterpret_cast<bf16x4 *>(dv + base + c) = v4;
            }
    }
}

// Query-stationary pass: each wave owns 32 queries; key tiles of KT in the
// band stream through LDS. Per tile: S^T = K~ Q^^T, P^T = exp(scale S^T - lse),
// dP^T = V~ dO^T, dS^T = P^T (dP^T - D), dQ^^T += K~^T dS^T.
// Epilogue: dq = scale R^T dQ^.
template <int DH, int KT, int ST>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(AttnArgs a, const bf16 *dO,
                                                              const float *lse2, const float *Dp,
                                                              int64_t Tp, bf16 *dq)
{
    constexpr int NF = DH / 16, NB = DH / 32, KB = KT / 32;
    constexpr int TE = KT * DH;
    constexpr int PER = 2 * TileDma<DH, KT, 4>::PER_WAVE;
    __shared__ __attribute__((aligned(1024))) bf16 lds[ST * 2 * TE];   // [stage][K, V]

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = (int)a.T, W = a.W;
    const int nqt = (T + 127) / 128;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = bid % nqt, bh = bid / nqt;
    const int h = bh % a.H;
    const int64_t b = bh / a.H;
    const int i0 = qt * 128, qw0 = i0 + 32 * w, qi = qw0 + l32;
    const int tok_stride = a.H * DH;
    const bf16 *kbase = a.kx + act_row(a, b, 0, h) * DH;
    const bf16 *vbase = a.vx + act_row(a, b, 0, h) * DH;

    const int klo = i0 - W + 1 > 0 ? i0 - W + 1 : 0;
    const int khi = i0 + 128 < T ? i0 + 128 : T;
    const int jstart = (klo / KT) * KT;
    const int nt = (khi - jstart + KT - 1) / KT;
    // This lane's query operands and statistics, waited for before any tile
    // load is issued: values still in flight at their first use inside the
    // loop would make the compiler wait for every load there (tiles included).
    bf16x8 qf[NF], df[NF];
    float lse_q = 0.0f, Dq = 0.0f;
    if (qi < T) {
        const int64_t base = act_row(a, b, qi, h) * DH;
        token_frags<DH>(a, a.qr + base, qi, g, false, 1.0f, qf);
        token_frags<DH>(a, dO + base, qi, g, false, 1.0f, df);
        lse_q = lse2[(int64_t)bh * Tp + qi];
        Dq = Dp[(int64_t)bh * Tp + qi];
    } else {
        zero_frags(qf, NF);
        zero_frags(df, NF);
    }
    wait_vmcnt<0>();

    auto issue = [&](int it) {
        bf16 *kt = lds + (it % ST) * 2 * TE;
        issue_kv_tile<DH, KT>(kbase, vbase, tok_stride, T, jstart + it * KT, kt, kt + TE, w, lane);
    };
#pragma unroll
    for (int s0 = 0; s0 < ST - 1; ++s0)
        if (s0 < nt) issue(s0);
    const float qscale = a.scale * kLog2e;
    f32x16 acc[NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;

    const bool active = qw0 < T;
    const int wlo = qw0 - W + 1;
    const int whi = qw0 + 31 < T - 1 ? qw0 + 31 : T - 1;

    for (int it = 0; it < nt; ++it) {
        pipeline_wait<ST, PER>(it, nt);
        if (it + ST - 1 < nt) issue(it + ST - 1);
        const int j0 = jstart + it * KT;
        if (!active || j0 > whi || j0 + KT - 1 < wlo) continue;
        const bf16 *kt = lds + (it % ST) * 2 * TE, *vt = kt + TE;

        f32x16 sc[KB], dp[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            bf16x8 kf[NF], vf[NF];   // every LDS read of the block issued before the products
#pragma unroll
            for (int s = 0; s < NF; ++s) {
                kf[s] = tile_rows<DH>(kt, kb, s, lane);
                vf[s] = tile_rows<DH>(vt, kb, s, lane);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) sc[kb][e] = dp[kb][e] = 0.0f;
#pragma unroll
            for (int s = 0; s < NF; ++s) {
                sc[kb] = mfma32(kf[s], qf[s], sc[kb]);
                dp[kb] = mfma32(vf[s], df[s], dp[kb]);
            }
        }
        const bool inside = (j0 + KT - 1 <= qw0) && (j0 >= qw0 + 31 - W + 1) && (j0 + KT - 1 < T);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = j0 + 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
                const bool ok = inside | ((key <= qi) & (key > qi - W) & (key < T));
                const float p = fast_exp2(sc[kb][e] * qscale - lse_q);
                dp[kb][e] = ok ? p * (dp[kb][e] - Dq) : 0.0f;
            }
        bf16x8 ktr[NB][2 * KB];
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int t = 0; t < 2 * KB; ++t) ktr[db][t] = tile_tr<DH>(kt, t, db, lane);
#pragma unroll
        for (int t = 0; t < 2 * KB; ++t) {
            const bf16x8 dsf = acc_to_operand(dp[t >> 1], t & 1);
#pragma unroll
            for (int db = 0; db < NB; ++db) acc[db] = mfma32(ktr[db][t], dsf, acc[db]);
        }
    }

    if (qi < T) {
        const int64_t base = act_row(a, b, qi, h) * DH;
        const float2 *cs = a.rope ? a.rope + (a.pos0 + qi) * (DH / 2) : nullptr;
        scale_rotate_back<NB>(acc, cs, g, a.scale);
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
static AttnArgs make_args(const Geom &g, const void *q, const void *qr, const void *kx,
                          const void *vx, const float2 *rope)
{
    AttnArgs a;
    a.q = static_cast<const bf16 *>(q);
    a.qr = static_cast<const bf16 *>(qr);
    a.kx = static_cast<const bf16 *>(kx);
    a.vx = static_cast<const bf16 *>(vx);
    a.rope = rope;
    a.B = g.B; a.T = g.T; a.H = g.H; a.W = g.W; a.pos0 = g.pos0; a.scale = g.scale;
    return a;
}

// Tile shapes and pipeline depths: forward and dQ stream K~/V~ tiles of
// kFwdKT keys through kFwdST stages; dK/dV streams 32-query tiles through
// kBwdST stages (kPairST in the wave-pair pass used for Dh = 128).
constexpr int kFwdKT = 32, kFwdST = 2, kDqKT = 32, kDqST = 2, kBwdST = 4, kPairST = 3;

void launch_attn_fwd_bf16(const Geom &g, const void *q, const void *kx, const void *vx,
                          const float2 *rope, void *o, float *lse, hipStream_t s)
{
    const AttnArgs a = make_args(g, q, nullptr, kx, vx, rope);
    const unsigned nwg = (unsigned)(g.B * g.H * ((g.T + 127) / 128));
    prof::Scope ts("attn_fwd", s);
    if (g.Dh == 128)
        hipLaunchKernelGGL((attn_fwd_kernel<128, kFwdKT, kFwdST>), dim3(nwg), dim3(256), 0, s, a,
                           static_cast<bf16 *>(o), lse);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<64, kFwdKT, kFwdST>), dim3(nwg), dim3(256), 0, s, a,
                           static_cast<bf16 *>(o), lse);
}

template <int DH>
static void launch_attn_bwd_t(const AttnArgs &a, const bf16 *o, const bf16 *dO, const float *lse,
                              void *dq, void *dk, void *dv, const BwdWorkspace &ws, int64_t rows,
                              unsigned nwg, bool entries, hipStream_t s)
{
    {
        const unsigned pre_blocks = (unsigned)((rows * (DH / 16) + 255) / 256);
        prof::Scope ts("attn_bwd_prep", s);
        hipLaunchKernelGGL(bwd_prep_kernel<DH>, dim3(pre_blocks), dim3(256), 0, s, o, dO, a.q, lse,
                           a.rope, static_cast<bf16 *>(ws.q_rot), ws.Dp, ws.lse2, rows, a.H, a.T,
                           ws.Tp, a.pos0);
    }
    {
        prof::Scope ts("attn_bwd_dkdv", s);
        if constexpr (DH == 128) {
            // one workgroup per 64 keys of a (sequence, head)
            const unsigned npw = (unsigned)(a.B * a.H * ((a.T + 63) / 64));
            if (entries)
                hipLaunchKernelGGL((attn_bwd_dkdv_pair_kernel<kPairST, false>), dim3(npw),
                                   dim3(256), 0, s, a, dO, ws.lse2, ws.Dp, ws.Tp,
                                   static_cast<bf16 *>(dk), static_cast<bf16 *>(dv));
            else
                hipLaunchKernelGGL((attn_bwd_dkdv_pair_kernel<kPairST, true>), dim3(npw),
                                   dim3(256), 0, s, a, dO, ws.lse2, ws.Dp, ws.Tp,
                                   static_cast<bf16 *>(dk), static_cast<bf16 *>(dv));
        } else if (entries) {
            hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DH, kBwdST, false>), dim3(nwg), dim3(256), 0,
                               s, a, dO, ws.lse2, ws.Dp, ws.Tp, static_cast<bf16 *>(dk),
                               static_cast<bf16 *>(dv));
        } else {
            hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DH, kBwdST, true>), dim3(nwg), dim3(256), 0, s,
                               a, dO, ws.lse2, ws.Dp, ws.Tp, static_cast<bf16 *>(dk),
                               static_cast<bf16 *>(dv));
        }
    }
    prof::Scope ts("attn_bwd_dq", s);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<DH, kDqKT, kDqST>), dim3(nwg), dim3(256), 0, s, a, dO,
                       ws.lse2, ws.Dp, ws.Tp, static_cast<bf16 *>(dq));
}

void launch_attn_bwd_bf16(const Geom &g, const void *q, const void *kx, const void *vx,
                          const void *o, const float *lse, const void *dO, void *dq, void *dk,
                          void *dv, const BwdWorkspace &ws, const float2 *rope, bool entries,
                          hipStream_t s)
{
    const AttnArgs a = make_args(g, q, ws.q_rot, kx, vx, rope);
    const int64_t rows = g.N() * g.H;
    const unsigned nwg = (unsigned)(g.B * g.H * ((g.T + 127) / 128));
    const bf16 *ob = static_cast<const bf16 *>(o);
    const bf16 *dOb = static_cast<const bf16 *>(dO);
    if (g.Dh == 128)
        launch_attn_bwd_t<128>(a, ob, dOb, lse, dq, dk, dv, ws, rows, nwg, entries, s);
    else
        launch_attn_bwd_t<64>(a, ob, dOb, lse, dq, dk, dv, ws, rows, nwg, entries, s);
}

}  // namespace mfma
}  // namespace maglev
