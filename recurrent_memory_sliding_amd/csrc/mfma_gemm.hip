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
// epilogue (dW). The gated form hands over gradients that already carry its
// gates and norm (no gate: s = 1).
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "mfma_kernels.hpp"
#include "profile.hpp"

namespace maglev {
namespace mfma {

// PIPE selects the main loop: true reads each K step's first fragments
// during the previous step's last MFMAs (one barrier inside the step); false
// keeps one barrier at the top of each step and fewer registers live, which
// the widest wave tiles need to stay within 256 VGPRs.
template <int BM_, int BN_, int WM_, int WN_, int STAGES_ = 3, bool PIPE_ = true>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 64, WM = WM_, WN = WN_;
    static constexpr int NT = WM_ * WN_ * 64;
    static constexpr int NW = WM_ * WN_;
    static constexpr int FM = BM_ / WM_ / 32;   // 32x32 blocks per wave along M
    static constexpr int FN = BN_ / WN_ / 32;
    static constexpr int STAGES = STAGES_;
    static constexpr bool PIPE = PIPE_;
};

// LDS layout of one operand tile, no padding, 16-byte chunks XOR-swizzled so
// that every read pass is free of bank conflicts:
//   K-major [R][64] (128-byte rows): chunk c of row r sits in slot c ^ ((r >> 1) & 7);
//     a ds_read_b128 pass (16 lanes, 16 rows, one chunk) then covers all 64 banks.
//   MN-major [64][R] (R >= 128): chunk c of row k sits in slot c ^ ((k & 3) << 2);
//     a transpose-read half wave (4 rows x 4 chunks) then covers all 64 banks.
template <bool KMAJOR, int R>
struct OpTile {
    static constexpr int ELEMS = R * 64;
    static constexpr int ROW = KMAJOR ? 64 : R;           // elements per LDS row
    static constexpr int CPR = ROW / 8;                    // chunks per row
    static constexpr int ROWS_PER_INSTR = 64 / CPR;        // rows one wave instruction fills
    static constexpr int INSTR = (KMAJOR ? R : 64) / ROWS_PER_INSTR;
    MAGLEV_DEV static int slot(int row, int c)
    {
        return KMAJOR ? (c ^ ((row >> 1) & 7)) : (c ^ ((row & 3) << 2));
    }
};

constexpr int kGemmSchedMfma = 0x8, kGemmSchedDsRead = 0x100;   // sched_group_barrier masks

// s_waitcnt lgkmcnt(0) with the other counters left alone (gfx9 encoding).
MAGLEV_DEV void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Source of rows that must read as zero (the shift's first row, K tails).
__device__ __attribute__((aligned(256))) bf16 g_zero_rows[64] = {};

MAGLEV_DEV bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

template <bool KMAJOR, int R>
MAGLEV_DEV bf16x8 read_frag(const bf16 *lds, int rb, int ks, int lane)
{
    using L = OpTile<KMAJOR, R>;
    if constexpr (KMAJOR) {
        const int r = rb * 32 + (lane & 31);
        const int c = 2 * ks + (lane >> 5);
        return *reinterpret_cast<const bf16x8 *>(lds + r * 64 + L::slot(r, c) * 8);
    } else {
        const int n0 = rb * 32 + 16 * ((lane >> 4) & 1);
        const int k0 = ks * 16 + 8 * (lane >> 5);
        const int j = lane & 15;
        const int n = n0 + 4 * (j & 3);
        const int c = n >> 3, e = n & 7;
        const int ka = k0 + (j >> 2), kb = ka + 4;
        const i16x4 lo = lds_read_tr16(lds + ka * R + L::slot(ka, c) * 8 + e);
        const i16x4 hi = lds_read_tr16(lds + kb * R + L::slot(kb, c) * 8 + e);
        return join_tr(lo, hi);
    }
}

// A problem with a `rowsum` member also wants, for every row, the sum over
// this tile's columns of the value its store_sum(m, n, x) returns; the tile
// writes it to rowsum[m * rs_ld + column tile].
template <class P, class = void>
struct HasRowSum : std::false_type {};
template <class P>
struct HasRowSum<P, std::void_t<decltype(std::declval<const P &>().rowsum)>> : std::true_type {};

// A problem with store4(m, t, n, v, split), which stores columns n .. n+3 of
// row m (N a multiple of 4), gets its accumulators transposed: the MFMA is
// issued with the operands swapped, so that a lane holds one row of each
// 32 x 32 block and runs of four consecutive columns (entries 4q .. 4q+3 are
// columns 8q + 4(lane / 32) + 0..3), and stores 8 or 16 bytes at a time.
template <class P, class = void>
struct HasStore4 : std::false_type {};
template <class P>
struct HasStore4<P, std::void_t<decltype(std::declval<const P &>().store4(
                        int64_t(), int64_t(), int64_t(), f32x4(), 0))>> : std::true_type {};

// Sums v[k] (k < 32) over the 32 lanes of each half wave with 31 exchanges:
// at distance D a lane keeps the half of its C live values selected by lane
// bit D and adds the partner's copy of that half. Afterwards v[0] of lane l
// holds the sum of value index l & 31. (One template level per distance, so
// every register index is a constant.)
template <int D, int C>
MAGLEV_DEV void transpose_sum_level(float (&v)[32], int lane)
{
    const bool hi = (lane & D) != 0;
#pragma unroll
    for (int k = 0; k < C / 2; ++k) {
        const float send = hi ? v[k] : v[C / 2 + k];
        const float keep = hi ? v[C / 2 + k] : v[k];
        v[k] = keep + __shfl_xor(send, D, 64);
    }
    if constexpr (D > 1) transpose_sum_level<D / 2, C / 2>(v, lane);
}
MAGLEV_DEV void half_wave_transpose_sum(float (&v)[32], int lane)
{
    transpose_sum_level<16, 32>(v, lane);
}

// C[M,N] = sum_k A(m,k) B(n,k) over k in this workgroup's split.
// P supplies: M, N, K; A_KMAJOR/B_KMAJOR; for a K-major operand x_ptr(row, k),
// the address of 8 elements along k, linear in k inside segments of x_kseg
// elements (0: one segment; otherwise a multiple of BK); for an MN-major
// operand (stored [k][col]) x_lin(k, col), the address of 8 elements along
// col, rows x_ld elements apart. The kernel only asks for rows < M / N and
// column chunks inside the matrix (it clamps); K tails read a zero page.
// Operands hold no zero rows:
// the shifts are applied in store(m, t, n, value, split), where t = m mod T.
// Pipeline: a ring of 3 LDS stages filled by direct global->LDS loads two
// stages ahead of the MFMA work; one barrier per 64-wide K step.
template <class Cfg, class P>
__global__ __launch_bounds__(Cfg::NT) void gemm_bf16(P p, int64_t kper, int group_m)
{
    using TA = OpTile<P::A_KMAJOR, Cfg::BM>;
    using TB = OpTile<P::B_KMAJOR, Cfg::BN>;
    constexpr int STAGE = TA::ELEMS + TB::ELEMS;
    static_assert(TA::INSTR % Cfg::NW == 0 && TB::INSTR % Cfg::NW == 0, "tile/wave mismatch");
    constexpr int IA = TA::INSTR / Cfg::NW, IB = TB::INSTR / Cfg::NW;   // DMA instructions per wave
    constexpr int PER_STAGE = IA + IB;
    __shared__ __attribute__((aligned(1024))) bf16 lds[Cfg::STAGES * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const int64_t ntn = (p.N + Cfg::BN - 1) / Cfg::BN;
    const int64_t ntm = (p.M + Cfg::BM - 1) / Cfg::BM;
    // Work item order: split-major; inside a split, groups of group_m tile rows
    // swept column by column. The dispatcher deals workgroups round-robin to
    // the 8 XCDs and xcd_remap gives each XCD a contiguous run of items, so
    // the workgroups resident on one XCD (one L2) share a few rows of A tiles
    // and a few columns of B tiles, and a split's K range stays on its XCDs.
    const int64_t item = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t per_split = ntm * ntn;
    const int split = (int)(item / per_split);
    const int64_t r = item % per_split;
    const int64_t gsz = (int64_t)group_m * ntn;
    const int64_t first_m = (r / gsz) * group_m;
    const int64_t gm = ntm - first_m < group_m ? ntm - first_m : group_m;
    const int64_t tm = first_m + (r % gsz) % gm, tn = (r % gsz) / gm;
    const int64_t m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
    const int64_t kb = (int64_t)split * kper;
    const int64_t ke = kb + kper < p.K ? kb + kper : p.K;
    const int nk = ke > kb ? (int)((ke - kb + Cfg::BK - 1) / Cfg::BK) : 0;

    // This lane's chunk of every DMA instruction: row inside the tile (its LDS
    // slot is fixed by the lane), the chunk it fetches (the swizzle is an
    // involution), and the global address at the current K step.
    const bf16 *pa[IA];
    const bf16 *pb[IB];
    int ka[IA], kbk[IB];   // k offset of the chunk inside the 64-wide step
    // Rows (K-major) or column chunks (MN-major) beyond M / N are clamped to the
    // last valid one: their products land in accumulator rows/columns the
    // epilogue never stores, so no lane ever needs a null check.
    auto a_addr = [&](int i, int64_t k0) -> const bf16 * {
        const int row = (wave * IA + i) * TA::ROWS_PER_INSTR + lane / TA::CPR;
        const int c = TA::slot(row, lane % TA::CPR);
        if constexpr (P::A_KMAJOR) {
            const int64_t r = m0 + row < p.M ? m0 + row : p.M - 1;
            return p.a_ptr(r, k0 + 8 * c);
        } else {
            const int64_t col = m0 + 8 * c < p.M ? m0 + 8 * c : p.M - 8;
            return p.a_lin(k0 + row, col);
        }
    };
    auto b_addr = [&](int i, int64_t k0) -> const bf16 * {
        const int row = (wave * IB + i) * TB::ROWS_PER_INSTR + lane / TB::CPR;
        const int c = TB::slot(row, lane % TB::CPR);
        if constexpr (P::B_KMAJOR) {
            const int64_t r = n0 + row < p.N ? n0 + row : p.N - 1;
            return p.b_ptr(r, k0 + 8 * c);
        } else {
            const int64_t col = n0 + 8 * c < p.N ? n0 + 8 * c : p.N - 8;
            return p.b_lin(k0 + row, col);
        }
    };
#pragma unroll
    for (int i = 0; i < IA; ++i) {
        const int row = (wave * IA + i) * TA::ROWS_PER_INSTR + lane / TA::CPR;
        ka[i] = P::A_KMAJOR ? 8 * TA::slot(row, lane % TA::CPR) : row;
        pa[i] = a_addr(i, kb);
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) {
        const int row = (wave * IB + i) * TB::ROWS_PER_INSTR + lane / TB::CPR;
        kbk[i] = P::B_KMAJOR ? 8 * TB::slot(row, lane % TB::CPR) : row;
        pb[i] = b_addr(i, kb);
    }
    const int64_t a_step = P::A_KMAJOR ? Cfg::BK : Cfg::BK * p.a_ld;
    const int64_t b_step = P::B_KMAJOR ? Cfg::BK : Cfg::BK * p.b_ld;
    // Next K at which an operand stored in segments (a_kseg / b_kseg elements,
    // multiples of BK) switches segment: its pointers are recomputed there.
    const int64_t a_seg = p.a_kseg > 0 ? p.a_kseg : 1, b_seg = p.b_kseg > 0 ? p.b_kseg : 1;
    int64_t a_next = p.a_kseg > 0 ? (kb / a_seg + 1) * a_seg : INT64_MAX;
    int64_t b_next = p.b_kseg > 0 ? (kb / b_seg + 1) * b_seg : INT64_MAX;

    // DMA of K step `it` into stage `buf` (the pointers are at step it), then
    // advance the pointers. Tails read the zero rows past ke.
    auto issue = [&](int it, int buf) {
        const int64_t k0 = kb + (int64_t)it * Cfg::BK;
        bf16 *sa = lds + buf * STAGE;
        bf16 *sb = sa + TA::ELEMS;
        const bool tail = k0 + Cfg::BK > ke;
        if (k0 == a_next) {
#pragma unroll
            for (int i = 0; i < IA; ++i) pa[i] = a_addr(i, k0);
            a_next += p.a_kseg;
        }
        if (k0 == b_next) {
#pragma unroll
            for (int i = 0; i < IB; ++i) pb[i] = b_addr(i, k0);
            b_next += p.b_kseg;
        }
        if (!tail) {
#pragma unroll
            for (int i = 0; i < IA; ++i) dma16(pa[i], sa + (wave * IA + i) * 512);
#pragma unroll
            for (int i = 0; i < IB; ++i) dma16(pb[i], sb + (wave * IB + i) * 512);
        } else {
#pragma unroll
            for (int i = 0; i < IA; ++i)
                dma16(k0 + ka[i] >= ke ? g_zero_rows : pa[i], sa + (wave * IA + i) * 512);
#pragma unroll
            for (int i = 0; i < IB; ++i)
                dma16(k0 + kbk[i] >= ke ? g_zero_rows : pb[i], sb + (wave * IB + i) * 512);
        }
#pragma unroll
        for (int i = 0; i < IA; ++i) pa[i] += a_step;
#pragma unroll
        for (int i = 0; i < IB; ++i) pb[i] += b_step;
    };

    constexpr bool TR = HasStore4<P>::value;   // accumulators hold row-per-lane blocks
    f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if constexpr (Cfg::PIPE) {
        // Fragment reads of sub-step ks (16 of the stage's 64 k) into buffer b.
        bf16x8 af[2][Cfg::FM], bfr[2][Cfg::FN];
        auto read_ks = [&](const bf16 *la, int ks, int b) {
            const bf16 *lb = la + TA::ELEMS;
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
                af[b][i] = read_frag<P::A_KMAJOR, Cfg::BM>(la, wm * Cfg::FM + i, ks, lane);
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j)
                bfr[b][j] = read_frag<P::B_KMAJOR, Cfg::BN>(lb, wn * Cfg::FN + j, ks, lane);
        };
        // The MFMAs of one sub-step with the reads of the next interleaved: two
        // LDS instructions (ds_read_b128, or one transpose-read pair) ahead of
        // each MFMA until the reads are out, so that they land while the rest of
        // the sub-step computes.
        constexpr int NREAD = Cfg::FM * (P::A_KMAJOR ? 1 : 2) + Cfg::FN * (P::B_KMAJOR ? 1 : 2);
        constexpr int NMFMA = Cfg::FM * Cfg::FN;
        auto mfma_ks = [&](int b) {
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
                    acc[i][j] = TR ? mfma32(bfr[b][j], af[b][i], acc[i][j]) : mfma32(af[b][i], bfr[b][j], acc[i][j]);
#pragma unroll
            for (int g = 0; g < (NREAD + 1) / 2 && g < NMFMA; ++g) {
                __builtin_amdgcn_sched_group_barrier(kGemmSchedDsRead, 2, 0);
                __builtin_amdgcn_sched_group_barrier(kGemmSchedMfma, 1, 0);
            }
            if constexpr (NMFMA > (NREAD + 1) / 2)
                __builtin_amdgcn_sched_group_barrier(kGemmSchedMfma, NMFMA - (NREAD + 1) / 2, 0);
        };

        // Pipeline: step s is loaded into stage s mod STAGES; the loads run
        // STAGES - 1 steps ahead of the MFMA work. The barrier of step it sits in
        // its last sub-step: there every wave's loads of step it+1 have landed
        // and no wave reads stage it any more, so it is refilled (step
        // it+STAGES) and the first fragments of step it+1 are read while the
        // last MFMAs of step it run.
#pragma unroll
        for (int s0 = 0; s0 < Cfg::STAGES; ++s0)
            if (s0 < nk) issue(s0, s0);
        if (nk > 0) {
            if (Cfg::STAGES >= 2 && nk >= Cfg::STAGES) wait_vmcnt<PER_STAGE * (Cfg::STAGES - 1)>();
            else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            read_ks(lds, 0, 0);
        }
        // (The last step is peeled off so that no join in the loop body makes the
        // compiler wait for the next step's fragments before this step's MFMAs.)
        auto step = [&](int it, auto last) {
            const bf16 *la = lds + (it % Cfg::STAGES) * STAGE;
#pragma unroll
            for (int ks = 0; ks < Cfg::BK / 16; ++ks) {
                const int cur = ks & 1;
                if (ks + 1 < Cfg::BK / 16) {
                    read_ks(la, ks + 1, cur ^ 1);
                } else if constexpr (!decltype(last)::value) {
                    // stage it+1 landed once at most the loads of steps
                    // it+2 .. it+STAGES-1 are in flight; this wave's reads of
                    // stage it have returned
                    if (Cfg::STAGES >= 3 && it + Cfg::STAGES - 1 < nk)
                        wait_vmcnt<PER_STAGE * (Cfg::STAGES >= 3 ? Cfg::STAGES - 2 : 0)>();
                    else wait_vmcnt<0>();
                    wait_lgkmcnt0();
                    __builtin_amdgcn_s_barrier();
                    if (it + Cfg::STAGES < nk) issue(it + Cfg::STAGES, it % Cfg::STAGES);
                    read_ks(lds + ((it + 1) % Cfg::STAGES) * STAGE, 0, cur ^ 1);
                }
                mfma_ks(cur);
            }
        };
        for (int it = 0; it + 1 < nk; ++it) step(it, std::false_type{});
        if (nk > 0) step(nk - 1, std::true_type{});
    } else {
        constexpr int AHEAD = Cfg::STAGES - 1;     // K steps in flight ahead of the MFMA work
#pragma unroll
        for (int s0 = 0; s0 < AHEAD; ++s0)
            if (s0 < nk) issue(s0, s0);
        for (int it = 0; it < nk; ++it) {
            // stage it has landed once at most (AHEAD - 1) later stages are still in flight
            if (AHEAD >= 2 && it + 1 < nk) wait_vmcnt<(AHEAD >= 2 ? PER_STAGE : 0)>();
            else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();            // every wave's share of stage it is in LDS,
                                                     // and stage it-1 is no longer being read
            if (it + AHEAD < nk) issue(it + AHEAD, (it + AHEAD) % Cfg::STAGES);
            const bf16 *la = lds + (it % Cfg::STAGES) * STAGE;
            const bf16 *lb = la + TA::ELEMS;
            bf16x8 af[2][Cfg::FM], bfr[2][Cfg::FN];
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
                af[0][i] = read_frag<P::A_KMAJOR, Cfg::BM>(la, wm * Cfg::FM + i, 0, lane);
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j)
                bfr[0][j] = read_frag<P::B_KMAJOR, Cfg::BN>(lb, wn * Cfg::FN + j, 0, lane);
#pragma unroll
            for (int ks = 0; ks < Cfg::BK / 16; ++ks) {
                const int cur = ks & 1;
                if (ks + 1 < Cfg::BK / 16) {
#pragma unroll
                    for (int i = 0; i < Cfg::FM; ++i)
                        af[cur ^ 1][i] = read_frag<P::A_KMAJOR, Cfg::BM>(la, wm * Cfg::FM + i, ks + 1, lane);
#pragma unroll
                    for (int j = 0; j < Cfg::FN; ++j)
                        bfr[cur ^ 1][j] = read_frag<P::B_KMAJOR, Cfg::BN>(lb, wn * Cfg::FN + j, ks + 1, lane);
                }
#pragma unroll
                for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                    for (int j = 0; j < Cfg::FN; ++j)
                        acc[i][j] = TR ? mfma32(bfr[cur][j], af[cur][i], acc[i][j])
                                       : mfma32(af[cur][i], bfr[cur][j], acc[i][j]);
            }
        }
    }

    // Epilogue: row index m and its position t = m mod T (from m0 mod T).
    const int g = lane >> 5;
    if constexpr (HasRowSum<P>::value) {
        // stores, and the per-row sums of store_sum's values over the tile's
        // valid columns: in-lane over j, across the half wave, across the WN
        // waves of a row band through LDS (the stages are no longer read once
        // every wave has passed the barrier)
        static_assert(Cfg::FM == 2, "row sums take 64 rows per wave");
        float v[32];
        auto values = [&](auto edge) {
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t m = m0 + (wm * Cfg::FM + i) * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                    float sum = 0.0f;
#pragma unroll
                    for (int j = 0; j < Cfg::FN; ++j) {
                        const int64_t n = n0 + (wn * Cfg::FN + j) * 32 + (lane & 31);
                        if (!decltype(edge)::value || (m < p.M && n < p.N))
                            sum += p.store_sum(m, n, acc[i][j][e]);
                    }
                    v[i * 16 + e] = sum;
                }
        };
        // a tile inside the matrix stores without per-element checks
        if (m0 + Cfg::BM <= p.M && n0 + Cfg::BN <= p.N) values(std::false_type{});
        else values(std::true_type{});
        half_wave_transpose_sum(v, lane);
        __syncthreads();
        float *rs = reinterpret_cast<float *>(lds);   // [WN][BM]
        const int k = lane & 31;
        const int r = (wm * Cfg::FM + (k >> 4)) * 32 + 8 * ((k >> 2) & 3) + 4 * g + (k & 3);
        rs[wn * Cfg::BM + r] = v[0];
        __syncthreads();
        for (int rr = tid; rr < Cfg::BM; rr += Cfg::NT) {
            const int64_t m = m0 + rr;
            if (m >= p.M) continue;
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < Cfg::WN; ++w) sum += rs[w * Cfg::BM + rr];
            p.rowsum[m * p.rs_ld + tn] = sum;
        }
    } else if constexpr (TR) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) {
            const int64_t m = m0 + (wm * Cfg::FM + i) * 32 + (lane & 31);
            if (m >= p.M) continue;
            const int64_t t = p.T > 0 ? m % p.T : 0;
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t n = n0 + (wn * Cfg::FN + j) * 32 + 8 * q + 4 * g;
                    if (n < p.N)
                        p.store4(m, t, n,
                                 f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                       acc[i][j][4 * q + 3]},
                                 split);
                }
        }
    } else {
        const int64_t t0 = p.T > 0 ? m0 % p.T : 0;
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = (wm * Cfg::FM + i) * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                const int64_t m = m0 + r;
                if (m >= p.M) continue;
                int64_t t = t0 + r;
                if (p.T > 0) while (t >= p.T) t -= p.T;
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j) {
                    const int64_t n = n0 + (wn * Cfg::FN + j) * 32 + (lane & 31);
                    if (n < p.N) p.store(m, t, n, acc[i][j][e], split);
                }
            }
    }
}

// Skinny product for M <= 64 rows (the decode step projects one memory row per
// stream): each workgroup owns 16 output columns, its four waves split K, and
// operands come straight from global memory (both K-contiguous) into
// v_mfma_f32_16x16x32_bf16 fragments; the four partial tiles are summed in LDS.
//   16x16x32 layout: operand lane l holds row/column l % 16 and K entries
//   8 (l / 16) .. +7; result lane l holds column l % 16, rows 4 (l / 16) .. +3.
template <class P>
__global__ __launch_bounds__(256) void gemm_skinny_bf16(P p)
{
    static_assert(P::A_KMAJOR && P::B_KMAJOR, "skinny path needs K-contiguous operands");
    __shared__ float red[4][4][64][4];     // [wave][row block][lane][e]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t kq = ((p.K + 127) / 128) * 32;              // K quarter, multiple of 32
    const int64_t k_lo = w * kq, k_hi = (k_lo + kq < p.K) ? k_lo + kq : p.K;
    const int r16 = lane & 15, kg = 8 * (lane >> 4);
    f32x4 acc[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t k0 = k_lo; k0 < k_hi; k0 += 32) {
        const int64_t k = k0 + kg;
        const bool kin = k < k_hi;
        const bool nin = kin && n0 + r16 < p.N;
        const bf16x8 bf = nin ? *reinterpret_cast<const bf16x8 *>(p.b_ptr(n0 + r16, k)) : zero8();
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const bool min_ = kin && 16 * rb + r16 < p.M;
            const bf16x8 af = min_ ? *reinterpret_cast<const bf16x8 *>(p.a_ptr(16 * rb + r16, k)) : zero8();
            acc[rb] = mfma16(af, bf, acc[rb]);
        }
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[w][rb][lane][e] = acc[rb][e];
    __syncthreads();
    // thread t sums one (row block, lane) slot over the four waves: 256 slots
    const int rb = tid >> 6, l = tid & 63;
    const int64_t n = n0 + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float x = red[0][rb][l][e] + red[1][rb][l][e] + red[2][rb][l][e] + red[3][rb][l][e];
        const int64_t m = 16 * rb + 4 * (l >> 4) + e;
        if (m < p.M && n < p.N) p.store(m, m % p.T, n, x, 0);
    }
}

// ---------------------------------------------------------------------------
// Problems
// ---------------------------------------------------------------------------
// The three products. Operands are plain row-major matrices; the one-token
// shift of the memory is applied where results are stored.
//
// Y [N_tok, 2HD] = m [N_tok, d] * [W_Km; W_Vm]^T. With shift 1, Y row (b,t)
// is the memory term of token (b,t+1): kmem[b,t+1] = Y[b,t] (t <= T-2) and
// kmem[b,0] = 0; with shift 0, kmem = Y.
struct ProjFwd {
    static constexpr bool A_KMAJOR = true, B_KMAJOR = true;
    const bf16 *m, *wk, *wv;
    bf16 *km, *vm;
    int64_t M, N, K, T;
    int HD, shift;
    static constexpr int64_t a_kseg = 0, b_kseg = 0, a_ld = 0, b_ld = 0;
    MAGLEV_DEV const bf16 *a_ptr(int64_t row, int64_t k) const { return m + row * K + k; }
    MAGLEV_DEV const bf16 *b_ptr(int64_t n, int64_t k) const
    {
        return n < HD ? wk + n * K + k : wv + (n - HD) * K + k;
    }
    MAGLEV_DEV const bf16 *a_lin(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV const bf16 *b_lin(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV void store(int64_t row, int64_t t, int64_t n, float x, int) const
    {
        bf16 *out = n < HD ? km : vm;
        const int64_t c = n < HD ? n : n - HD;
        if (shift) {
            if (t == 0) out[row * HD + c] = f2bf(0.0f);
            if (t + 1 < T) out[(row + 1) * HD + c] = f2bf(x);
        } else {
            out[row * HD + c] = f2bf(x);
        }
    }
    // four columns n .. n+3 (HD is a multiple of 4: they lie on one side)
    MAGLEV_DEV void store4(int64_t row, int64_t t, int64_t n, f32x4 x, int) const
    {
        bf16 *out = n < HD ? km : vm;
        const int64_t c = n < HD ? n : n - HD;
        const bf16x4 v{f2bf(x[0]), f2bf(x[1]), f2bf(x[2]), f2bf(x[3])};
        if (shift) {
            if (t == 0) *reinterpret_cast<bf16x4 *>(out + row * HD + c) = bf16x4{};
            if (t + 1 < T) *reinterpret_cast<bf16x4 *>(out + (row + 1) * HD + c) = v;
        } else {
            *reinterpret_cast<bf16x4 *>(out + row * HD + c) = v;
        }
    }
};

// dX [N_tok, d] = G [N_tok, 2HD] * Ws [2HD, d], G = [dk | dv] (k segments of
// HD), Ws = s_h-scaled [W_Km; W_Vm] stored transposed, [d][2HD], so that both
// operands are K-major. dX row (b,t) is the gradient of the memory row
// m'[b,t-1] (t >= 1).
struct ProjBwdDm {
    static constexpr bool A_KMAJOR = true, B_KMAJOR = true;
    const bf16 *dk, *dv, *wt;
    float *dm;
    int64_t M, N, K, T;
    int HD;
    bool acc;
    int64_t a_kseg;
    static constexpr int64_t b_kseg = 0, a_ld = 0, b_ld = 0;
    MAGLEV_DEV const bf16 *a_ptr(int64_t row, int64_t k) const
    {
        return k < HD ? dk + row * HD + k : dv + row * HD + (k - HD);
    }
    MAGLEV_DEV const bf16 *b_ptr(int64_t n, int64_t k) const { return wt + n * K + k; }
    MAGLEV_DEV const bf16 *a_lin(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV const bf16 *b_lin(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV void store(int64_t row, int64_t t, int64_t n, float x, int) const
    {
        // m'[T-1] feeds no key: its injection gradient is zero (written here
        // unless accumulating); row t's product lands on m'[t-1].
        if (t == T - 1 && !acc) dm[row * N + n] = 0.0f;
        if (t == 0) return;
        float *p = dm + (row - 1) * N + n;
        *p = acc ? *p + x : x;
    }
    MAGLEV_DEV void store4(int64_t row, int64_t t, int64_t n, f32x4 x, int) const
    {
        if (t == T - 1 && !acc) *reinterpret_cast<f32x4 *>(dm + row * N + n) = f32x4{};
        if (t == 0) return;
        f32x4 *p = reinterpret_cast<f32x4 *>(dm + (row - 1) * N + n);
        *p = acc ? *p + x : x;
    }
};

// dW partial [2HD, d] = sum over tokens u of G[u+1]^T m'[u] (u = 0 .. N_tok-2),
// one split of that range. A = G rows shifted by one token, stored [u][2HD]
// (columns < HD from dk, the rest from dv); B = m' stored [u][d]. The pairs
// that cross a sequence boundary (u = b T - 1) are subtracted in dw_reduce.
struct ProjBwdDw {
    static constexpr bool A_KMAJOR = false, B_KMAJOR = false;
    const bf16 *dk, *dv, *m;
    float *part;      // [ksplit][2HD][d]
    int64_t M, N, K, T;
    int HD;
    int64_t a_ld, b_ld;
    static constexpr int64_t a_kseg = 0, b_kseg = 0;
    MAGLEV_DEV const bf16 *a_ptr(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV const bf16 *b_ptr(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV const bf16 *a_lin(int64_t u, int64_t r) const
    {
        return r < HD ? dk + (u + 1) * HD + r : dv + (u + 1) * HD + (r - HD);
    }
    MAGLEV_DEV const bf16 *b_lin(int64_t u, int64_t e) const { return m + u * N + e; }
    MAGLEV_DEV void store(int64_t r, int64_t, int64_t e, float x, int split) const
    {
        part[((int64_t)split * M + r) * N + e] = x;
    }
    MAGLEV_DEV void store4(int64_t r, int64_t, int64_t e, f32x4 x, int split) const
    {
        *reinterpret_cast<f32x4 *>(part + ((int64_t)split * M + r) * N + e) = x;
    }
};

// Loss-head products ([V, d] head U, N_tok rows):
//   logits  C[n, v] = cap tanh((m U^T)[n, v] / cap)    A = m [N,d], B = U [V,d], both K-major
//   dm      dm[n, e] = sum_v dz[n, v] U[v, e]           A = dz [N,V] K-major, B = U MN-major
//   dU      dU[v, e] (+)= sum_n dz[n, v] m[n, e]        A = dz MN-major, B = m MN-major
//   the logits product also sums exp(c) over each tile's columns per row: c
//   lies in [-cap, cap] with cap <= 64, so exp(c) is finite and normal in
//   float32 and the row's log-sum-exp needs no running maximum.
struct LmLogits {
    static constexpr bool A_KMAJOR = true, B_KMAJOR = true;
    const bf16 *m, *u;
    float *out;
    float *rowsum;
    int64_t rs_ld;
    int64_t M, N, K, T;
    float cap, inv_cap2;   // cap, 2 / cap
    static constexpr int64_t a_kseg = 0, b_kseg = 0, a_ld = 0, b_ld = 0;
    MAGLEV_DEV const bf16 *a_ptr(int64_t row, int64_t k) const { return m + row * K + k; }
    MAGLEV_DEV const bf16 *b_ptr(int64_t n, int64_t k) const { return u + n * K + k; }
    MAGLEV_DEV const bf16 *a_lin(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV const bf16 *b_lin(int64_t, int64_t) const { return nullptr; }
    // c = cap tanh(x / cap), tanh(y) = 1 - 2 / (exp(2y) + 1) (exp(2y) may
    // overflow to inf for large y, which gives tanh = 1 exactly); returns exp(c)
    MAGLEV_DEV float store_sum(int64_t row, int64_t n, float x) const
    {
        const float c = cap - 2.0f * cap * __builtin_amdgcn_rcpf(__expf(x * inv_cap2) + 1.0f);
        out[row * N + n] = c;
        return __expf(c);
    }
};
struct LmDm {
    static constexpr bool A_KMAJOR = true, B_KMAJOR = false;
    const bf16 *dz, *u;
    float *dm;
    int64_t M, N, K, T;
    int64_t b_ld;
    static constexpr int64_t a_kseg = 0, b_kseg = 0, a_ld = 0;
    MAGLEV_DEV const bf16 *a_ptr(int64_t row, int64_t k) const { return dz + row * K + k; }
    MAGLEV_DEV const bf16 *b_ptr(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV const bf16 *a_lin(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV const bf16 *b_lin(int64_t k, int64_t n) const { return u + k * b_ld + n; }
    MAGLEV_DEV void store(int64_t row, int64_t, int64_t n, float x, int) const { dm[row * N + n] = x; }
    MAGLEV_DEV void store4(int64_t row, int64_t, int64_t n, f32x4 x, int) const
    {
        *reinterpret_cast<f32x4 *>(dm + row * N + n) = x;
    }
};
// dm = dz U with U read from its transposed copy ut [d][V], so that both
// operands are K-major (256 x 320 tiles take K-major operands only).
struct LmDmT {
    static constexpr bool A_KMAJOR = true, B_KMAJOR = true;
    const bf16 *dz, *ut;
    float *dm;
    int64_t M, N, K, T;
    static constexpr int64_t a_kseg = 0, b_kseg = 0, a_ld = 0, b_ld = 0;
    MAGLEV_DEV const bf16 *a_ptr(int64_t row, int64_t k) const { return dz + row * K + k; }
    MAGLEV_DEV const bf16 *b_ptr(int64_t n, int64_t k) const { return ut + n * K + k; }
    MAGLEV_DEV const bf16 *a_lin(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV const bf16 *b_lin(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV void store(int64_t row, int64_t, int64_t n, float x, int) const { dm[row * N + n] = x; }
    MAGLEV_DEV void store4(int64_t row, int64_t, int64_t n, f32x4 x, int) const
    {
        *reinterpret_cast<f32x4 *>(dm + row * N + n) = x;
    }
};
struct LmDu {
    static constexpr bool A_KMAJOR = false, B_KMAJOR = false;
    const bf16 *dz, *m;
    float *du;
    int64_t M, N, K, T;
    int64_t a_ld, b_ld;
    bool acc;
    static constexpr int64_t a_kseg = 0, b_kseg = 0;
    MAGLEV_DEV const bf16 *a_ptr(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV const bf16 *b_ptr(int64_t, int64_t) const { return nullptr; }
    MAGLEV_DEV const bf16 *a_lin(int64_t k, int64_t col) const { return dz + k * a_ld + col; }
    MAGLEV_DEV const bf16 *b_lin(int64_t k, int64_t col) const { return m + k * b_ld + col; }
    MAGLEV_DEV void store(int64_t r, int64_t, int64_t e, float x, int) const
    {
        float *p = du + r * N + e;
        *p = acc ? *p + x : x;
    }
    MAGLEV_DEV void store4(int64_t r, int64_t, int64_t e, f32x4 x, int) const
    {
        f32x4 *p = reinterpret_cast<f32x4 *>(du + r * N + e);
        *p = acc ? *p + x : x;
    }
};

// Tile configurations, chosen by timing the three products at the d20 shape
// (N_tok = 16384, d = 1280, 10 x 128 heads) with random operands: two LDS
// stages and 8 waves per workgroup, so that each SIMD has two or more waves to
// cover LDS and barrier latency (one wave per SIMD left the matrix cores idle
// most of the time).
// The projection and dX have a short reduction (1280, 2560), so per-tile
// start-up and stores weigh: 256 x 320 tiles (wave tile 64 x 160, 0.7 KB of
// LDS reads per MFMA) make exactly two rounds of the 256 CUs for the
// projection (N = 2560) and one for dX (N = 1280). Smaller problems, which
// would leave CUs idle with them, take 128 x 128 tiles (two workgroups a CU).
using ProjBigCfg = TileCfg<256, 320, 4, 2, 2, false>;
using ProjCfg = TileCfg<128, 128, 2, 4, 2>;    // wave tile 64 x 32
using DwCfg = TileCfg<256, 256, 2, 4, 2>;      // wave tile 128 x 64, split over tokens
// At most 64 rows (decode: one memory row per stream) against many output
// columns (every layer's stacked weights): one 64-row tile, weights streamed
// once. The product is bound by the latency of the weight loads: three stages
// of 64 x 256 tiles (one workgroup a CU) stream the 131 MB of 20 d20 layers
// in 30 µs, two stages of 64 x 128 (three a CU) in 32.5 µs.
using WideCfg = TileCfg<64, 256, 1, 4, 3, false>;   // wave tile 64 x 64

// Whether an M x N product fills at least one round of the CUs with 256 x 320 tiles.
bool proj_big_tiles(int64_t M, int64_t N)
{
    return ((M + ProjBigCfg::BM - 1) / ProjBigCfg::BM) * ((N + ProjBigCfg::BN - 1) / ProjBigCfg::BN) >= 256;
}

template <class Cfg, class P>
static void run_gemm(const P &p, int ksplit, int64_t kper, hipStream_t s, const char *name,
                     int group_m)
{
    const int64_t ntm = (p.M + Cfg::BM - 1) / Cfg::BM;
    const int64_t ntn = (p.N + Cfg::BN - 1) / Cfg::BN;
    if (group_m > ntm) group_m = (int)ntm;
    prof::Scope ts(name, s, prof::Scope::Attach{});
    hipExtLaunchKernelGGL((gemm_bf16<Cfg, P>), dim3((unsigned)(ntm * ntn * ksplit)), dim3(Cfg::NT), 0,
                          s, ts.start(), ts.stop(), 0, p, kper, group_m);
}

// out[c][r] = in[r][c] for a bf16 [R][C] matrix (C and R multiples of 8),
// one workgroup per 64 x 64 block staged through LDS, so that both the reads
// and the writes are 16-byte runs.
__global__ __launch_bounds__(256) void transpose_bf16(const bf16 *in, bf16 *out, int64_t R, int C)
{
    __shared__ float tile[64][65];
    const int64_t r0 = (int64_t)blockIdx.y * 64;
    const int c0 = blockIdx.x * 64;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int c = threadIdx.x + 256 * q;   // 512 chunks of 8: row c / 8, chunk c % 8
        const int rr = c >> 3, cc = c0 + 8 * (c & 7);
        float x[8] = {};
        if (r0 + rr < R && cc < C) load8(in + (r0 + rr) * C + cc, x);
#pragma unroll
        for (int u = 0; u < 8; ++u) tile[8 * (c & 7) + u][rr] = x[u];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int c = threadIdx.x + 256 * q;   // output row c0 + c / 8, chunk c % 8 of r
        const int cc = c >> 3;
        const int64_t r = r0 + 8 * (c & 7);
        if (c0 + cc >= C || r >= R) continue;
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = tile[cc][8 * (c & 7) + u];
        store8(out + (int64_t)(c0 + cc) * R + r, x);
    }
}

// Loss-head products, timed at N = 16384, d = 1280, V = 65536 with random
// operands: the logits (a short reduction, d = 1280, like the projection) on
// 256 x 320 tiles with the single-barrier loop (2.95 ms against 3.28 ms for
// 256 x 256), dU on 256 x 256 tiles with 8 waves (a 128 x 64 block per wave),
// dm on 128 x 128 (d = 1280 gives only 320 tiles of 256 x 256); all three
// sweep small groups of tile rows (2 to 8) so that the workgroups on one XCD
// share their A and B tiles in its L2.
using LmLogitsCfg = TileCfg<256, 320, 4, 2, 2, false>;
using LmDuCfg = TileCfg<256, 256, 2, 4, 2>;

int64_t lm_logits_col_tiles(int64_t V) { return (V + LmLogitsCfg::BN - 1) / LmLogitsCfg::BN; }

void launch_lm_logits_bf16(int64_t N, int64_t V, int d, float cap, const void *m, const void *u,
                           float *logits, float *rowsum, hipStream_t s)
{
    LmLogits p;
    p.m = static_cast<const bf16 *>(m);
    p.u = static_cast<const bf16 *>(u);
    p.out = logits;
    p.rowsum = rowsum;
    p.rs_ld = lm_logits_col_tiles(V);
    p.M = N; p.N = V; p.K = d; p.T = 0; p.cap = cap; p.inv_cap2 = 2.0f / cap;
    run_gemm<LmLogitsCfg>(p, 1, p.K, s, "lm_logits", 8);
}

void launch_lm_dm_bf16(int64_t N, int64_t V, int d, const void *dz, const void *u, void *ut,
                       float *dm, hipStream_t s)
{
    if (proj_big_tiles(N, d)) {
        // 256 x 320 tiles over K-major operands: U transposed once into ut
        // [d][V]; then each row block of dz is read by d / 320 column tiles
        // (four at d = 1280) instead of d / 128, in one round of the CUs
        {
            prof::Scope ts("lm_dm_transpose", s);
            hipLaunchKernelGGL(transpose_bf16, dim3((unsigned)((d + 63) / 64), (unsigned)((V + 63) / 64)),
                               dim3(256), 0, s, static_cast<const bf16 *>(u),
                               static_cast<bf16 *>(ut), V, d);
        }
        LmDmT p;
        p.dz = static_cast<const bf16 *>(dz);
        p.ut = static_cast<const bf16 *>(ut);
        p.dm = dm;
        p.M = N; p.N = d; p.K = V; p.T = 0;
        run_gemm<ProjBigCfg>(p, 1, p.K, s, "lm_dm", 8);
        return;
    }
    LmDm p;
    p.dz = static_cast<const bf16 *>(dz);
    p.u = static_cast<const bf16 *>(u);
    p.dm = dm;
    p.M = N; p.N = d; p.K = V; p.T = 0; p.b_ld = d;
    run_gemm<ProjCfg>(p, 1, p.K, s, "lm_dm", 2);
}

void launch_lm_du_bf16(int64_t N, int64_t V, int d, const void *dz, const void *m, float *du,
                       bool acc, hipStream_t s)
{
    LmDu p;
    p.dz = static_cast<const bf16 *>(dz);
    p.m = static_cast<const bf16 *>(m);
    p.du = du;
    p.M = V; p.N = d; p.K = N; p.T = 0; p.a_ld = V; p.b_ld = d; p.acc = acc;
    run_gemm<LmDuCfg>(p, 1, p.K, s, "lm_du", 2);
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
    if (p.M <= 64 && p.N >= 8192) {
        run_gemm<WideCfg>(p, 1, p.K, s, "proj_fwd_wide", 1);
    } else if (p.M <= 64) {
        prof::Scope ts("proj_fwd_skinny", s);
        hipLaunchKernelGGL(gemm_skinny_bf16<ProjFwd>, dim3((unsigned)((p.N + 15) / 16)), dim3(256), 0,
                           s, p);
    } else if (proj_big_tiles(p.M, p.N)) {
        run_gemm<ProjBigCfg>(p, 1, p.K, s, "proj_fwd", 4);
    } else {
        run_gemm<ProjCfg>(p, 1, p.K, s, "proj_fwd", 16);
    }
}

// Transposed s_h-scaled copy of [W_Km; W_Vm]: out[e][r] = s_h(r) W[r][e]
// (rows r < HD from W_Km, the rest from W_Vm; s_h = 1 when gate is null).
// One workgroup per 64 x 64 block (2HD is a multiple of 128, d of 16), staged
// through LDS so that both the reads and the writes are 16-byte runs.
__global__ __launch_bounds__(256) void scale_weights_t(const bf16 *wk, const bf16 *wv,
                                                       const float *gate, bf16 *out, int HD,
                                                       int Dh, int d)
{
    __shared__ float tile[64][65];
    const int r0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
    const int R = 2 * HD;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int c = threadIdx.x + 256 * q;   // 512 chunks of 8: row c / 8, chunk c % 8
        const int rr = c >> 3, e = e0 + 8 * (c & 7);
        const int r = r0 + rr;
        float x[8] = {};
        if (e < d) {
            const bf16 *src = r < HD ? wk + (int64_t)r * d : wv + (int64_t)(r - HD) * d;
            load8(src + e, x);
            const float sg = gate ? gate_sigmoid(gate[(r < HD ? r : r - HD) / Dh]) : 1.0f;
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] *= sg;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) tile[8 * (c & 7) + u][rr] = x[u];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int c = threadIdx.x + 256 * q;   // output row e0 + c / 8, chunk c % 8 of r
        const int ee = c >> 3, e = e0 + ee;
        if (e >= d) continue;
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = tile[ee][8 * (c & 7) + u];
        store8(out + (int64_t)e * R + r0 + 8 * (c & 7), x);
    }
}

// One workgroup per row r of [dW_Km; dW_Vm], 8 columns a thread:
//   G[r,:] = sum of the split partials (fixed order) - boundary pairs,
//   dW[r,:] (+)= s_h G[r,:]   (s_h = 1 when gate is null),
//   rowdot[r] = <W[r,:], G[r,:]>  when rowdot is not null.
// The boundary pairs are G[bT]^T m'[bT-1] for b = 1 .. B-1: the shifted
// product pairs the first token of a sequence with the last memory row of the
// previous one. rowdot is the row's share of the sigma gate's gradient:
// sum_t <kmem_t, dk_t> = sum_t <W_Km x_t, dk_t> = <W_Km, sum_t dk_t x_t^T>.
__global__ __launch_bounds__(256) void dw_reduce(const float *part, int ksplit, int HD, int Dh,
                                                 int d, int64_t B, int64_t T, const bf16 *dk,
                                                 const bf16 *dv, const bf16 *m, const bf16 *wk,
                                                 const bf16 *wv, const float *gate, float *dwk,
                                                 float *dwv, float *rowdot, bool acc)
{
    __shared__ float red[4];
    const int r = blockIdx.x;
    const int64_t tot = 2 * (int64_t)HD * d;
    const int rr = r < HD ? r : r - HD;
    const bf16 *G = r < HD ? dk : dv;
    const bf16 *Wr = (r < HD ? wk : wv) + (int64_t)rr * d;
    float *out = (r < HD ? dwk : dwv) + (int64_t)rr * d;
    const float sg = gate ? gate_sigmoid(gate[rr / Dh]) : 1.0f;
    float dot = 0.0f;
    for (int e = threadIdx.x * 8; e < d; e += blockDim.x * 8) {   // d is a multiple of 16
        const int64_t i = (int64_t)r * d + e;
        float x[8], y[8];
        load8(part + i, x);
        for (int sp = 1; sp < ksplit; ++sp) {
            load8(part + sp * tot + i, y);
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] += y[u];
        }
        for (int64_t b = 1; b < B; ++b) {
            const float gv = bf2f(G[(b * T) * HD + rr]);
            load8(m + (b * T - 1) * d + e, y);
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] -= gv * y[u];
        }
        if (rowdot) {
            load8(Wr + e, y);
#pragma unroll
            for (int u = 0; u < 8; ++u) dot += y[u] * x[u];
        }
        if (acc) load8(out + e, y);
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = acc ? y[u] + x[u] * sg : x[u] * sg;
        store8(out + e, x);
    }
    if (!rowdot) return;
    dot = wave_sum(dot);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = dot;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
        rowdot[r] = t;
    }
}

int dw_ksplit(const Geom &g)
{
    // 256 x 256 tiles of dW (one workgroup per CU at a time): split the token
    // range so that the grid is close to one workgroup per CU, keeping >= 1024
    // tokens per split.
    const int64_t tiles = ((2 * (int64_t)g.HD() + 255) / 256) * ((g.d + 255) / 256);
    int64_t ks = 256 / tiles;
    const int64_t max_by_k = (g.N() + 1023) / 1024;
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
        prof::Scope ts("proj_bwd_scale_w", s);
        hipLaunchKernelGGL(scale_weights_t, dim3((unsigned)((g.d + 63) / 64), (unsigned)(2 * HD / 64)),
                           dim3(256), 0, s, static_cast<const bf16 *>(wk),
                           static_cast<const bf16 *>(wv), gate, wsc, HD, g.Dh, g.d);
    }
    {
        ProjBwdDm p;
        p.dk = static_cast<const bf16 *>(dk);
        p.dv = static_cast<const bf16 *>(dv);
        p.wt = wsc;
        p.dm = dm_prime;
        p.M = g.N(); p.N = g.d; p.K = 2 * (int64_t)HD; p.T = g.T;
        p.HD = HD;
        p.acc = (acc & 1u) != 0;
        p.a_kseg = HD;
        if (proj_big_tiles(p.M, p.N)) run_gemm<ProjBigCfg>(p, 1, p.K, s, "proj_bwd_dm", 4);
        else run_gemm<ProjCfg>(p, 1, p.K, s, "proj_bwd_dm", 2);
    }
    {
        ProjBwdDw p;
        p.dk = static_cast<const bf16 *>(dk);
        p.dv = static_cast<const bf16 *>(dv);
        p.m = static_cast<const bf16 *>(m_prime);
        p.part = ws.dW_part;
        p.M = 2 * (int64_t)HD; p.N = g.d; p.K = g.N() - 1; p.T = 0;
        p.HD = HD;
        p.a_ld = HD;
        p.b_ld = g.d;
        const int ks = ws.ksplit;
        int64_t kper = (p.K + ks - 1) / ks;
        kper = (kper + 63) / 64 * 64;
        // Tiles in row-major order inside each split: the workgroups of one XCD
        // then cover few row tiles of dk/dv (and every column tile of m'), so
        // its L2 fetches each slice of the operands about once (about 195 MB a
        // d20 launch against 242 MB column by column, 126 MB algorithmic).
        run_gemm<DwCfg>(p, ks, kper, s, "proj_bwd_dw", 1);
        const int per_row = (g.d / 8 + 63) / 64 * 64;
        prof::Scope ts("proj_bwd_dw_reduce", s);
        hipLaunchKernelGGL(dw_reduce, dim3((unsigned)(2 * HD)), dim3(per_row < 256 ? per_row : 256),
                           0, s, ws.dW_part, ks, HD, g.Dh, g.d, g.B, g.T, p.dk, p.dv, p.m,
                           static_cast<const bf16 *>(wk), static_cast<const bf16 *>(wv), gate, dWk,
                           dWv, gate ? ws.rowdot : nullptr, (acc & 2u) != 0);
    }
}

}  // namespace mfma
}  // namespace maglev
