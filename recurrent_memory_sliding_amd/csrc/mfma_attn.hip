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
// owning 32 rows; v_mfma_f32_32x32x16_bf16 with fp32 accumulation (the dK/dV
// pass for Dh = 128: 16 keys a wave, v_mfma_f32_16x16x32_bf16, so that three
// workgroups share a CU and no values cross between waves). Scores are
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
#include <type_traits>

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

// Third dword of a raw buffer descriptor for untyped buffer instructions on
// gfx9-family chips: a valid 32-bit data format, no swizzle, no index
// stride (offsets at or beyond num_records are dropped stores).
constexpr int kBufferWord3 = 0x00020000;
// Cache policy of a buffer access: nontemporal (streamed past the caches the
// re-read tiles live in).
constexpr int kNontemporal = 2;
typedef int i32x2 __attribute__((ext_vector_type(2)));

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
// Byte offsets of this lane's chunks of a wave's DMA instructions inside a
// tile of KT token rows, rows tok_stride elements apart.
template <int DH, int KT>
MAGLEV_DEV void kv_tile_offsets(int tok_stride, int w, int lane,
                                unsigned (&voff)[TileDma<DH, KT, 4>::PER_WAVE])
{
    using Dma = TileDma<DH, KT, 4>;
#pragma unroll
    for (int i = 0; i < Dma::PER_WAVE; ++i) {
        const int ins = w * Dma::PER_WAVE + i;
        const int r = Dma::row(ins, lane);
        voff[i] = (unsigned)(r * tok_stride + Dma::chunk(r, lane) * 8) * 2u;
    }
}

// DMA of the K~ and V~ tiles of keys j0 .. j0+KT-1 (four waves). A tile inside
// the sequence is read through buffer descriptors of its KT rows (uniform
// registers) at the lane offsets voff, with no vector instructions; a tile
// reaching past T reads those rows from the zero page.
template <int DH, int KT>
MAGLEV_DEV void issue_kv_tile(const bf16 *kbase, const bf16 *vbase, int tok_stride, int T, int j0,
                              bf16 *kt, bf16 *vt, int w, int lane,
                              const unsigned (&voff)[TileDma<DH, KT, 4>::PER_WAVE])
{
    using Dma = TileDma<DH, KT, 4>;
    if (j0 + KT <= T) {
        const int64_t toff = (int64_t)j0 * tok_stride;
        const unsigned bytes = (unsigned)(KT * tok_stride) * 2u;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16 *>(kbase + toff), (short)0, bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16 *>(vbase + toff), (short)0, bytes, kBufferWord3);
#pragma unroll
        for (int i = 0; i < Dma::PER_WAVE; ++i) {
            const int ins = w * Dma::PER_WAVE + i;
            dma16_buf(rk, voff[i], kt + ins * 512);
            dma16_buf(rv, voff[i], vt + ins * 512);
        }
        return;
    }
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

// Calls f(it + U, U) for U = U0 .. N-1 while it + U < nt, each U a
// compile-time constant.
template <int U, int N, class F>
MAGLEV_DEV void unrolled_steps(int it, int nt, F &f)
{
    if constexpr (U < N) {
        if (it + U >= nt) return;
        f(it + U, std::integral_constant<int, U>{});
        unrolled_steps<U + 1, N>(it, nt, f);
    }
}

// Tile order of a pass that sweeps nt tiles of ts tokens, the first at token
// `first`, in rotated order: step it takes the tile whose absolute index is
// congruent to it modulo nt. The forward's query blocks of one (sequence,
// head) that share a key tile (five at W = 512) then read it at about the
// same step, while it is still in L2, instead of one after another as each
// sweeps its own band from its start: the six (sequence, head) pairs resident
// on one XCD hold 6 MB of K~/V~, more than its 4 MB L2. The dK/dV pass for
// Dh = 128 sweeps its query tiles the same way (three workgroups a CU keep
// three pairs' Q^ / dO resident per XCD; the rotation took its fetched bytes
// from 283 to 215 MB a launch at d20, its time unchanged). The dQ pass keeps
// the plain order: its resident K~ tiles fit in L2.
struct TileSweep {
    int nt, phase;
    MAGLEV_DEV TileSweep(int first, int nt_, int ts) : nt(nt_)
    {
        phase = nt > 0 ? (nt - (first / ts) % nt) % nt : 0;
    }
    MAGLEV_DEV int rel(int it) const
    {
        const int r = it + phase;
        return r < nt ? r : r - nt;
    }
};

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
    const TileSweep sweep(jstart, nt, KT);
    // The query operands are complete before any tile load is issued (see the
    // dQ pass for why). They are bf16(R q) unscaled, the operand the backward
    // recomputes the scores from, so that its probabilities are the ones whose
    // log-sum-exp this pass records; the softmax scale (times log2 e) is
    // applied to the float32 scores inside the exponent's fma.
    bf16x8 qf[NF];
    if (qi < T) token_frags<DH>(a, a.q + act_row(a, b, qi, h) * DH, qi, g, true, 1.0f, qf);
    else zero_frags(qf, NF);
    wait_vmcnt<0>();
    const float c2 = a.scale * kLog2e;   // scores -> log2 units

    unsigned voff[TileDma<DH, KT, 4>::PER_WAVE];
    kv_tile_offsets<DH, KT>(tok_stride, w, lane, voff);
    // tile `it` into stage `buf` (it mod ST)
    auto issue = [&](int it, int buf) {
        bf16 *kt = lds + buf * 2 * TE;
        issue_kv_tile<DH, KT>(kbase, vbase, tok_stride, T, jstart + sweep.rel(it) * KT, kt, kt + TE,
                              w, lane, voff);
    };
#pragma unroll
    for (int s0 = 0; s0 < ST - 1; ++s0)
        if (s0 < nt) issue(s0, s0);

    f32x16 acc[NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    const bool active = qw0 < T;
    const int wlo = qw0 - W + 1;
    const int whi = qw0 + 31 < T - 1 ? qw0 + 31 : T - 1;
    // keys qi - band + 1 .. qi are seen by query qi (none past T: its row is
    // not stored)
    const unsigned band = qi < T ? (unsigned)W : 0u;

    // Step `it`; U = it mod ST is a compile-time constant, so that every LDS
    // address of the step is a lane base plus an immediate offset.
    auto step = [&](int it, auto u) {
        constexpr int U = decltype(u)::value;
        pipeline_wait<ST, PER>(it, nt);
        if (it + ST - 1 < nt) issue(it + ST - 1, (U + ST - 1) % ST);
        const int j0 = jstart + sweep.rel(it) * KT;
        if (!active || j0 > whi || j0 + KT - 1 < wlo) return;
        const bf16 *kt = lds + U * 2 * TE, *vt = kt + TE;

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
            // key j is in query qi's band iff 0 <= qi - j < band
            const int d0 = qi - j0 - 4 * g;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if ((unsigned)(d0 - 32 * kb - 8 * (e >> 2) - (e & 3)) >= band) sc[kb][e] = -INFINITY;
        }
        // running maximum of the raw scores (c2 > 0 keeps the order)
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][e]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2((m_run - m_use) * c2);
        const float mc = m_use * c2;
        float rs = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = fast_exp2(fmaf(sc[kb][e], c2, -mc));
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
    };
    for (int it = 0; it < nt; it += ST) unrolled_steps<0, ST>(it, nt, step);

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
        if (g == 0 && lse) lse[(b * a.H + h) * a.T + qi] = (m_run * c2 + log2f(l_run)) * kLn2;
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

// Key-stationary pass with one wave per 16 keys (Dh = 128): four waves, 64
// keys a workgroup, each wave computing all of its keys' work alone with
// v_mfma_f32_16x16x32_bf16, so that no values cross between waves and the
// only shared state is the ring of 32-query Q^ / dO tiles (and their lse2 / D
// rows) in LDS. Per tile a wave forms S = Q^ K~^T and dP = dO V~^T (lane l:
// key l % 16, queries 16 qb + 4 (l / 16) + i), P = exp(scale S - lse) on the
// band, dS = P (dP - D), then dV^T += dO^T P and dK^T += Q^^T dS with the
// probabilities' query order matched by the transposed reads (lane l of the
// result: key l % 16, channels 16 cb + 4 (l / 16) + i). dS, rounded to bf16 as
// the dK product takes it, is stored for the dQ pass in tiles of 32 keys x
// 32 queries (2 KB; a wave writes the kilobyte of its 16 keys in its own lane
// order, one 16-byte store a lane).
namespace k16 {
// Swizzle of the Q^ / dO tiles: chunk c of row r sits in slot c ^ swz(r),
// with bits 2-3 of swz from r mod 4 and bits 0-1 a bijection of (r / 4) mod 4
// that puts rows 4 apart into opposite halves of bit 1. The transposed reads
// (rows 4g .. 4g+3 of two chunks for g = 0, 1 or 2, 3 in a half-wave pass)
// then meet every slot once. The row reads take chunk s + 4 (lane / 16) in
// step s; with chunk 4 s + lane / 16 instead, the same swizzle measured 3.9
// bank-conflict cycles a ds_read_b128 (SQ_LDS_BANK_CONFLICT), and the 32-row
// passes' swizzle conflicts on these transposed reads.
MAGLEV_DEV int swz(int r)
{
    const int g = (r >> 2) & 3;
    return ((r & 3) << 2) | ((g & 1) << 1) | (g >> 1);
}
MAGLEV_DEV int off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 3); }
constexpr int TE = 32 * 128;            // elements of one 32-row tile
constexpr int STATS = 4 * 64;           // floats: one 64-float slot a wave
constexpr int SE = 2 * TE + 2 * STATS;  // bf16 elements of one stage
constexpr int PER = 5;                  // vector memory operations a wave issues per stage
}  // namespace k16

template <int ST, bool ROTATE>
__global__ __launch_bounds__(256, 3) void attn_bwd_dkdv_k16_kernel(AttnArgs a, const bf16 *dO,
                                                                    const float *lse2,
                                                                    const float *Dp, int64_t Tp,
                                                                    bf16 *dk, bf16 *dv, bf16 *dso,
                                                                    int nK, int nt32)
{
    static_assert(ST >= 2, "at least one tile in flight");
    constexpr int DH = 128, QT = 32, PER = k16::PER;
    __shared__ __attribute__((aligned(1024))) bf16 lds[ST * k16::SE];   // [stage][Q^, dO, stats]

    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = (int)a.T, W = a.W;
    const int nkt = (T + 63) / 64;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = bid % nkt, bh = bid / nkt;
    const int h = bh % a.H;
    const int64_t b = bh / a.H;
    const int j0 = kt * 64, kw0 = j0 + 16 * w, kj = kw0 + l16;
    const float qscale = a.scale * kLog2e;
    const int tok_stride = a.H * DH;
    const bf16 *qbase = a.qr + act_row(a, b, 0, h) * DH;
    const bf16 *obase = dO + act_row(a, b, 0, h) * DH;
    const float *lrow = lse2 + (int64_t)bh * Tp;
    const float *drow = Dp + (int64_t)bh * Tp;

    const int qend = j0 + 63 + W < T ? j0 + 63 + W : T;   // exclusive
    // queries kj .. kj + band - 1 see key kj: band = min(W, T - kj), 0 past T
    const unsigned band = kj < T ? (unsigned)(W < T - kj ? W : T - kj) : 0u;
    const int nt = (qend - j0 + QT - 1) / QT;
    // step it takes the query tile whose absolute index is congruent to it
    // modulo nt, so that the workgroups sharing a tile read it at about the
    // same step (the sums over tiles are order-free)
    const TileSweep sweep(j0, nt, QT);

    // This lane's key row of K~ and of V~ as B operands: fragment s holds
    // chunk s + 4 (lane / 16), channels 8 s + 32 (lane / 16) .. +7 (the order
    // of the channels inside a product is free; this one keeps the row reads
    // below free of bank conflicts). Complete before any tile load.
    bf16x8 kf[4], vf[4];
    if (kj < T) {
        const bf16 *ks = a.kx + act_row(a, b, kj, h) * DH;
        const bf16 *vs = a.vx + act_row(a, b, kj, h) * DH;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            kf[s] = *reinterpret_cast<const bf16x8 *>(ks + 8 * s + 32 * g4);
            vf[s] = *reinterpret_cast<const bf16x8 *>(vs + 8 * s + 32 * g4);
        }
    } else {
        zero_frags(kf, 4);
        zero_frags(vf, 4);
    }
    wait_vmcnt<0>();

    // DMA: instruction ins (0..7) of a tile fills rows 4 ins .. +3; the lane's
    // LDS slot is fixed, its source chunk is slot ^ swz(row). This wave issues
    // instructions 2w and 2w + 1 of the Q^ tile and of the dO tile, then its
    // own 64-float statistics slot (lse2 of the tile's 32 queries, then D).
    unsigned voff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 4 * (2 * w + i) + (lane >> 4);
        voff[i] = (unsigned)(r * tok_stride + ((l16 ^ k16::swz(r)) << 3)) * 2u;
    }
    const float *ssrc = lane < 32 ? lrow + lane : drow + (lane - 32);
    auto issue = [&](int it, int buf) {
        const int i0 = j0 + sweep.rel(it) * QT;
        bf16 *qt = lds + buf * k16::SE, *ot = qt + k16::TE;
        float *st = reinterpret_cast<float *>(ot + k16::TE) + 64 * w;
        if (i0 + QT <= T) {
            const int64_t toff = (int64_t)i0 * tok_stride;
            const unsigned bytes = (unsigned)(QT * tok_stride) * 2u;
            const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<bf16 *>(qbase + toff), (short)0, bytes, kBufferWord3);
            const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<bf16 *>(obase + toff), (short)0, bytes, kBufferWord3);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ins = 2 * w + i;
                dma16_buf(rq, voff[i], qt + ins * 512);
                dma16_buf(ro, voff[i], ot + ins * 512);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ins = 2 * w + i;
                const int r = 4 * ins + (lane >> 4);
                const int qi = i0 + r;
                const int64_t o = (int64_t)qi * tok_stride + ((l16 ^ k16::swz(r)) << 3);
                dma16(qi < T ? qbase + o : g_attn_zero, qt + ins * 512);
                dma16(qi < T ? obase + o : g_attn_zero, ot + ins * 512);
            }
        }
        // rows are padded to Tp (a multiple of 32), so the tile's 32 values exist
        dma4(ssrc + i0, st);
    };

    f32x4 dva[8], dka[8];   // dV^T, dK^T: channels 16 cb + 4 (lane / 16) + i of key kj
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) dva[cb] = dka[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s0 = 0; s0 < ST - 1; ++s0)
        if (s0 < nt) issue(s0, s0);

    // dS of this wave: half w % 2 (keys 16 (w % 2) .. +15) of the 32-key
    // tile kw0 / 32, stored in the lanes' own order so that one 16-byte store
    // a lane writes the half's whole kilobyte: lane 16 g4 + l16 (key l16 of
    // the half; queries 4 g4 .. +3, then 16 + 4 g4 .. +3) takes 16-byte slot
    // 16 g4 + (l16 ^ 4 g4) (the XOR keeps the dQ pass's transposed reads of
    // the tile free of bank conflicts)
    const int kt32 = kw0 >> 5;
    const int ds_voff = 1024 * (w & 1) + 16 * (16 * g4 + (l16 ^ (4 * g4)));
    int s1 = 0, s2 = 0;   // dS stores issued in the last and the one before
    auto step = [&](int it, auto u) {
        constexpr int U = decltype(u)::value;
        // tile it has landed once at most the operations issued after it are
        // outstanding: step it-2's stores, tile it+1, step it-1's stores
        // (loads and stores complete in issue order)
        switch (s1 + s2 + (it + 1 < nt ? PER : 0)) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case PER: wait_vmcnt<PER>(); break;
        case PER + 1: wait_vmcnt<PER + 1>(); break;
        default: wait_vmcnt<PER + 2>(); break;
        }
        __builtin_amdgcn_s_barrier();
        if (it + ST - 1 < nt) issue(it + ST - 1, (U + ST - 1) % ST);   // the stage tile it-1 used
        const int i0 = j0 + sweep.rel(it) * QT;
        const bf16 *qt = lds + U * k16::SE, *ot = qt + k16::TE;
        const float *st = reinterpret_cast<const float *>(ot + k16::TE) + 64 * w;
        // dS for the dQ pass, for the query tiles it reads (the first at the
        // key tile's own queries, nK in all)
        const int jj = (i0 >> 5) - kt32;
        const bool stored = dso && jj >= 0 && jj < nK;
        s2 = s1;
        s1 = stored ? 1 : 0;
        // S and dP: blocks qb of 16 queries, 4 K steps of 32 channels (lane
        // group g4 holds chunk s + 4 g4 of its row, as the B operands)
        f32x4 sa[2], pa[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            sa[qb] = pa[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int r = 16 * qb + l16;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(qt + k16::off(r, s + 4 * g4));
                sa[qb] = mfma16(aq, kf[s], sa[qb]);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 ao = *reinterpret_cast<const bf16x8 *>(ot + k16::off(r, s + 4 * g4));
                pa[qb] = mfma16(ao, vf[s], pa[qb]);
            }
        }
        f32x4 l2[2], dd[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            l2[qb] = *reinterpret_cast<const f32x4 *>(st + 16 * qb + 4 * g4);
            dd[qb] = *reinterpret_cast<const f32x4 *>(st + 32 + 16 * qb + 4 * g4);
        }
        // every (query, key) pair of the wave's block in the band: no mask
        const bool interior = (i0 >= kw0 + 15) & (i0 + QT - 1 - kw0 < W) & (i0 + QT - 1 < T);
        bf16x8 pf, dsf;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float p = fast_exp2(sa[qb][i] * qscale - l2[qb][i]);
                if (!interior) {
                    // query q is in key kj's band iff 0 <= q - kj < band
                    const bool ok = (unsigned)(i0 + 16 * qb + 4 * g4 + i - kj) < band;
                    p = ok ? p : 0.0f;
                }
                pf[4 * qb + i] = f2bf(p);
                dsf[4 * qb + i] = f2bf(p * (pa[qb][i] - dd[qb][i]));
            }
        if (stored) {
            bf16 *tile = dso + (((int64_t)bh * nt32 + kt32) * nK + jj) * 1024;
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc(tile, (short)0, 2048, kBufferWord3);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, dsf), rs, ds_voff, 0,
                                                   kNontemporal);
        }
        // dV^T += dO^T P, dK^T += Q^^T dS: A operand of block cb is column
        // 16 cb + l16 at queries 4 g4 + 0..3 and 16 + 4 g4 + 0..3 (the order of
        // the probabilities' entries), from two transposed reads whose lane j
        // addresses row 4 g4 + j / 4 (+16) at column 16 cb + 4 (j % 4)
        const int ra = 4 * g4 + (l16 >> 2);
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
            const int n = 16 * cb + 4 * (l16 & 3);
            const int c = n >> 3, e = n & 7;
            const bf16x8 ao = join_tr(lds_read_tr16(ot + k16::off(ra, c) + e),
                                      lds_read_tr16(ot + k16::off(ra + 16, c) + e));
            const bf16x8 aq = join_tr(lds_read_tr16(qt + k16::off(ra, c) + e),
                                      lds_read_tr16(qt + k16::off(ra + 16, c) + e));
            dva[cb] = mfma16(ao, pf, dva[cb]);
            dka[cb] = mfma16(aq, dsf, dka[cb]);
        }
    };
    for (int it = 0; it < nt; it += ST) unrolled_steps<0, ST>(it, nt, step);

    // Epilogue: lane holds key kj, channels 16 cb + 4 g4 + i; dk = scale R^T dK~
    // (pairs c, c + 64 are blocks cb, cb + 4 of the same lane)
    if (kj < T) {
        const int64_t base = act_row(a, b, kj, h) * DH;
        const float2 *cs = (a.rope && ROTATE) ? a.rope + (a.pos0 + kj) * (DH / 2) : nullptr;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            f32x4 &lo = dka[cb], &hi = dka[cb + 4];
            if (cs) {
                const float *t = reinterpret_cast<const float *>(cs + 16 * cb + 4 * g4);
                const f32x4 t0 = *reinterpret_cast<const f32x4 *>(t);
                const f32x4 t1 = *reinterpret_cast<const f32x4 *>(t + 4);
                const float cx[4] = {t0[0], t0[2], t1[0], t1[2]};
                const float sy[4] = {t0[1], t0[3], t1[1], t1[3]};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = lo[i] * a.scale, y = hi[i] * a.scale;
                    lo[i] = x * cx[i] + y * sy[i];
                    hi[i] = -x * sy[i] + y * cx[i];
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lo[i] *= a.scale;
                    hi[i] *= a.scale;
                }
            }
        }
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
            bf16x4 k4, v4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                k4[i] = f2bf(dka[cb][i]);
                v4[i] = f2bf(dva[cb][i]);
            }
            *reinterpret_cast<bf16x4 *>(dk + base + 16 * cb + 4 * g4) = k4;
            *reinterpret_cast<bf16x4 *>(dv + base + 16 * cb + 4 * g4) = v4;
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

    unsigned voff[TileDma<DH, KT, 4>::PER_WAVE];
    kv_tile_offsets<DH, KT>(tok_stride, w, lane, voff);
    auto issue = [&](int it) {
        bf16 *kt = lds + (it % ST) * 2 * TE;
        issue_kv_tile<DH, KT>(kbase, vbase, tok_stride, T, jstart + it * KT, kt, kt + TE, w, lane, voff);
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

// Transposed operand in natural key order: reduction rows 16 tt + 8 g + {0..7}
// (g = lane / 32), column 32 db + (lane % 32) -- the layout of an operand
// whose 8 K entries are consecutive rows of the tile.
MAGLEV_DEV bf16x8 tile_tr_nat(const bf16 *t, int tt, int db, int lane)
{
    constexpr int DH = 128;
    const int g = lane >> 5, j = lane & 15;
    const int n = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
    const int c = n >> 3, e = n & 7;
    const int ra = 16 * tt + 8 * g + (j >> 2);
    const i16x4 lo = lds_read_tr16(t + tile_off<DH>(ra, c) + e);
    const i16x4 hi = lds_read_tr16(t + tile_off<DH>(ra + 4, c) + e);
    return join_tr(lo, hi);
}

// Query-stationary dQ pass from the stored dS tiles (Dh = 128): each wave
// owns 32 queries (one query tile), the workgroup 128; the K~ tiles of the
// workgroup's band and each wave's own dS tile of the same 32 keys stream
// through LDS in ST stages. Per tile: dQ^^T += K~^T dS^T (8 products), no
// scores, no softmax. Epilogue as the recomputing pass: dq = scale R^T dQ^.
// A dS tile sits in LDS as stored: two halves of 16 keys, each as the dK/dV
// pass's lanes held it (16-byte slot 16a + (key ^ 4a) holds one key's
// queries 4a .. 4a+3 and 16 + 4a .. +3). Its operand (query column, 8
// consecutive keys) comes from transposed reads of those 8-byte query runs;
// the XOR puts the 16 runs a lane group reads in 16 different bank groups.
template <int ST>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_ds_kernel(AttnArgs a, const bf16 *ds, int nK,
                                                                 int nt32, bf16 *dq)
{
    constexpr int DH = 128, NB = DH / 32, KT = 32;
    constexpr int TE = KT * DH;            // K~ tile
    constexpr int DSE = 32 * 32;           // one wave's dS tile
    constexpr int SE = TE + 4 * DSE;       // one stage
    using Dma = TileDma<DH, KT, 4>;
    constexpr int PER = Dma::PER_WAVE + 2;  // vector memory ops a wave issues per stage
    __shared__ __attribute__((aligned(1024))) bf16 lds[ST * SE];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = (int)a.T, W = a.W;
    const int nqt = (T + 127) / 128;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = bid % nqt, bh = bid / nqt;
    const int h = bh % a.H;
    const int64_t b = bh / a.H;
    const int i0 = qt * 128, qw0 = i0 + 32 * w, qi = qw0 + l32;
    const int wqt = qw0 >> 5;                                          // this wave's query tile
    const int wkt_lo = (qw0 - W + 1 > 0 ? qw0 - W + 1 : 0) >> 5;     // its first key tile
    const bool active = qw0 < T;
    const int tok_stride = a.H * DH;
    const bf16 *kbase = a.kx + act_row(a, b, 0, h) * DH;
    const bf16 *dsbase = ds + (int64_t)bh * nt32 * nK * DSE;

    const int klo = i0 - W + 1 > 0 ? i0 - W + 1 : 0;
    const int khi = i0 + 128 < T ? i0 + 128 : T;
    const int jstart = (klo / KT) * KT;
    const int nt = (khi - jstart + KT - 1) / KT;

    // K~ tile of the workgroup (two instructions a wave) and this wave's dS
    // tile of the same keys (two more: 16 rows of 64 bytes each), read from
    // the zero page where the wave has no such tile.
    // A K~ tile inside the sequence and a dS tile the wave has are read
    // through buffer descriptors (uniform registers, built per tile) at fixed
    // lane offsets; otherwise rows beyond T, or the whole dS tile, come from
    // the zero page.
    unsigned voff[Dma::PER_WAVE];
    kv_tile_offsets<DH, KT>(tok_stride, w, lane, voff);
    const unsigned ds_off = (unsigned)lane * 16u;
    auto issue = [&](int it, int buf) {   // buf = it mod ST
        bf16 *st = lds + buf * SE;
        const int j0 = jstart + it * KT;
        if (j0 + KT <= T) {
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<bf16 *>(kbase + (int64_t)j0 * tok_stride), (short)0,
                (unsigned)(KT * tok_stride) * 2u, kBufferWord3);
#pragma unroll
            for (int i = 0; i < Dma::PER_WAVE; ++i)
                dma16_buf(rk, voff[i], st + (w * Dma::PER_WAVE + i) * 512);
        } else {
#pragma unroll
            for (int i = 0; i < Dma::PER_WAVE; ++i) {
                const int ins = w * Dma::PER_WAVE + i;
                const int r = Dma::row(ins, lane);
                const int c = Dma::chunk(r, lane);
                const int j = j0 + r;
                dma16(j < T ? kbase + (int64_t)j * tok_stride + c * 8 : g_attn_zero, st + ins * 512);
            }
        }
        const int kt = j0 >> 5;
        const bool have = active && kt >= wkt_lo && kt <= wqt;
        bf16 *dst = st + TE + w * DSE;
        if (have) {
            const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<bf16 *>(dsbase + ((int64_t)kt * nK + (wqt - kt)) * DSE), (short)0,
                DSE * 2, kBufferWord3);
            dma16_buf_once(rd, ds_off, dst);
            dma16_buf_once(rd, ds_off + 1024u, dst + 512);
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) dma16(g_attn_zero, dst + i * 512);
        }
    };
#pragma unroll
    for (int s0 = 0; s0 < ST - 1; ++s0)
        if (s0 < nt) issue(s0, s0);

    f32x16 acc[NB];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;

    // Step `it`; U = it mod ST is a compile-time constant, so that every LDS
    // address of the step is a lane base plus an immediate offset.
    auto step = [&](int it, auto u) {
        constexpr int U = decltype(u)::value;
        pipeline_wait<ST, PER>(it, nt);
        if (it + ST - 1 < nt) issue(it + ST - 1, (U + ST - 1) % ST);
        const int kt = (jstart >> 5) + it;
        if (!active || kt < wkt_lo || kt > wqt) return;
        const bf16 *kt_lds = lds + U * SE;
        const bf16 *ds_lds = kt_lds + TE + w * DSE;
        bf16x8 ktr[NB][2], dsf[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            // keys 16t + 8g + (0..3) and (4..7) of query column l32. Half t of
            // the tile holds key kk of the half and queries 4a .. 4a+3 (and
            // 16 + 4a .. +3) in 16-byte slot 16a + (kk ^ 4a); lane j of a
            // group of 16 addresses key 8g + j/4 (+4) of queries 4(j%4) .. +3,
            // the half of the slot that holds query block (lane / 16) % 2.
            const int j = lane & 15, qa = j & 3, kk = 8 * g + (j >> 2);
            const bf16 *p = ds_lds + 512 * t + 4 * ((lane >> 4) & 1);
            dsf[t] = join_tr(lds_read_tr16(p + 8 * (16 * qa + (kk ^ (4 * qa)))),
                             lds_read_tr16(p + 8 * (16 * qa + ((kk + 4) ^ (4 * qa)))));
#pragma unroll
            for (int db = 0; db < NB; ++db) ktr[db][t] = tile_tr_nat(kt_lds, t, db, lane);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int db = 0; db < NB; ++db) acc[db] = mfma32(ktr[db][t], dsf[t], acc[db]);
    };
    for (int it = 0; it < nt; it += ST) unrolled_steps<0, ST>(it, nt, step);

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
// kBwdST stages (kK16ST in the 16-keys-a-wave pass used for Dh = 128).
constexpr int kFwdKT = 32, kFwdST = 2, kDqKT = 32, kDqST = 2, kBwdST = 4, kDqDsST = 3,
              kK16ST = 3;

void launch_attn_fwd_bf16(const Geom &g, const void *q, const void *kx, const void *vx,
                          const float2 *rope, void *o, float *lse, hipStream_t s)
{
    const AttnArgs a = make_args(g, q, nullptr, kx, vx, rope);
    const unsigned nwg = (unsigned)(g.B * g.H * ((g.T + 127) / 128));
    prof::Scope ts("attn_fwd", s, prof::Scope::Attach{});
    if (g.Dh == 128)
        hipExtLaunchKernelGGL((attn_fwd_kernel<128, kFwdKT, kFwdST>), dim3(nwg), dim3(256), 0, s,
                              ts.start(), ts.stop(), 0, a, static_cast<bf16 *>(o), lse);
    else
        hipExtLaunchKernelGGL((attn_fwd_kernel<64, kFwdKT, kFwdST>), dim3(nwg), dim3(256), 0, s,
                              ts.start(), ts.stop(), 0, a, static_cast<bf16 *>(o), lse);
}

template <int DH>
static void launch_attn_bwd_t(const AttnArgs &a, const bf16 *o, const bf16 *dO, const float *lse,
                              void *dq, void *dk, void *dv, const BwdWorkspace &ws, int64_t rows,
                              unsigned nwg, bool entries, hipStream_t s)
{
    {
        const unsigned pre_blocks = (unsigned)((rows * (DH / 16) + 255) / 256);
        prof::Scope ts("attn_bwd_prep", s, prof::Scope::Attach{});
        hipExtLaunchKernelGGL(bwd_prep_kernel<DH>, dim3(pre_blocks), dim3(256), 0, s, ts.start(),
                              ts.stop(), 0, o, dO, a.q, lse, a.rope,
                              static_cast<bf16 *>(ws.q_rot), ws.Dp, ws.lse2, rows, a.H, a.T,
                              ws.Tp, a.pos0);
    }
    {
        prof::Scope ts("attn_bwd_dkdv", s, prof::Scope::Attach{});
        if constexpr (DH == 128) {
            // one workgroup per 64 keys of a (sequence, head)
            const unsigned npw = (unsigned)(a.B * a.H * ((a.T + 63) / 64));
            bf16 *dso = static_cast<bf16 *>(ws.ds);
            if (entries)
                hipExtLaunchKernelGGL((attn_bwd_dkdv_k16_kernel<kK16ST, false>), dim3(npw),
                                      dim3(256), 0, s, ts.start(), ts.stop(), 0, a, dO, ws.lse2,
                                      ws.Dp, ws.Tp, static_cast<bf16 *>(dk),
                                      static_cast<bf16 *>(dv), dso, ws.ds_tiles, ws.nt32);
            else
                hipExtLaunchKernelGGL((attn_bwd_dkdv_k16_kernel<kK16ST, true>), dim3(npw),
                                      dim3(256), 0, s, ts.start(), ts.stop(), 0, a, dO, ws.lse2,
                                      ws.Dp, ws.Tp, static_cast<bf16 *>(dk),
                                      static_cast<bf16 *>(dv), dso, ws.ds_tiles, ws.nt32);
        } else if (entries) {
            hipExtLaunchKernelGGL((attn_bwd_dkdv_kernel<DH, kBwdST, false>), dim3(nwg), dim3(256),
                                  0, s, ts.start(), ts.stop(), 0, a, dO, ws.lse2, ws.Dp, ws.Tp,
                                  static_cast<bf16 *>(dk), static_cast<bf16 *>(dv));
        } else {
            hipExtLaunchKernelGGL((attn_bwd_dkdv_kernel<DH, kBwdST, true>), dim3(nwg), dim3(256),
                                  0, s, ts.start(), ts.stop(), 0, a, dO, ws.lse2, ws.Dp, ws.Tp,
                                  static_cast<bf16 *>(dk), static_cast<bf16 *>(dv));
        }
    }
    prof::Scope ts("attn_bwd_dq", s, prof::Scope::Attach{});
    if (DH == 128 && ws.ds)
        hipExtLaunchKernelGGL((attn_bwd_dq_ds_kernel<kDqDsST>), dim3(nwg), dim3(256), 0, s,
                              ts.start(), ts.stop(), 0, a, static_cast<const bf16 *>(ws.ds),
                              ws.ds_tiles, ws.nt32, static_cast<bf16 *>(dq));
    else
        hipExtLaunchKernelGGL((attn_bwd_dq_kernel<DH, kDqKT, kDqST>), dim3(nwg), dim3(256), 0, s,
                              ts.start(), ts.stop(), 0, a, dO, ws.lse2, ws.Dp, ws.Tp,
                              static_cast<bf16 *>(dq));
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
