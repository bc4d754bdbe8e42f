// gated_mix.hip -- the gated mixing form and its backward.
//
// Method: Maglev summary on paper.rainbus.top ("Maglev：滑动窗口循环记忆"),
// section 方法步骤详情: the recurrent key is the RMS-normalised projection of
// the shifted memory, and each layer mixes it with the local features through
// channel-wise gates g = 2 sigmoid(a) (neutral value 1 at a = 0); section
// 前置知识: both keys are rotated before the mix. Per token row of H*Dh
// channels (p = pos0 + t, kp = W_Km m'_{t-1}, rms = sqrt(mean(kp^2) + eps)):
//   kn   = kp / rms
//   k~   = g_kl (.) R_p k + g_kr (.) R_p kn,     v~ = g_vl (.) v + g_vr (.) vmem
// Backward, from the gradients dk~, dv~ of the mixed entries:
//   dk   = R_p^T (g_kl (.) dk~),   dkn = R_p^T (g_kr (.) dk~)
//   dkp  = (dkn - kn mean(dkn (.) kn)) / rms      (mean over the H*Dh row)
//   dv   = g_vl (.) dv~,           dvmem = g_vr (.) dv~
//   d/da = 2 sigmoid(a)(1 - sigmoid(a)) * sum over tokens of
//          dk~ (.) R k | dk~ (.) R kn | dv~ (.) v | dv~ (.) vmem.
//
// Layout of the work: one workgroup walks a contiguous range of token rows;
// each thread owns one chunk pair of the row (8 channels c..c+7 of a head and
// their rotation partners c+Dh/2..; H*Dh <= 4096, so at most 256 threads) for
// the whole range, so it keeps its gate-gradient
// partial sums in registers (the gate values sit in LDS). The row reductions
// (sum of squares; in the backward also mean of dkn*kn, in the same pass) are
// workgroup sums.
// Everything is HBM-bound streaming: 16-byte loads and stores per lane.
#include "common.hpp"
#include "internal.hpp"
#include "profile.hpp"

namespace maglev {

namespace {

constexpr int kGatedFwdRows = 16;  // token rows per workgroup in the forward mix (d20: 1024
                                    // workgroups, all resident at once)

MAGLEV_DEV float two_sigmoid(float a) { return 2.0f / (1.0f + __expf(-a)); }

// Sum over one row group of nw waves (wi: this wave's index inside it); every
// thread of the group receives the total. `red` holds one float per wave;
// callers alternate buffers between consecutive sums so that one barrier per
// sum suffices, and every thread of the workgroup calls it (it holds the
// workgroup barrier).
MAGLEV_DEV float group_sum(float x, float *red, int nw, int wi)
{
    x = wave_sum(x);
    if ((threadIdx.x & 63) == 0) red[wi] = x;
    __syncthreads();
    float t = 0.0f;
    for (int i = 0; i < nw; ++i) t += red[i];
    return t;
}

// Rotation of the 8 pairs (lo[e], hi[e]) by the table entries cs[0..7];
// inverse applies R^T.
MAGLEV_DEV void rotate_pairs(float *lo, float *hi, const float2 *cs, bool inverse)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float c = cs[e].x, sn = inverse ? -cs[e].y : cs[e].y;
        const float x0 = lo[e], x1 = hi[e];
        lo[e] = x0 * c - x1 * sn;
        hi[e] = x0 * sn + x1 * c;
    }
}

// Channel geometry of thread `cp`'s chunk pair inside an H*Dh row.
template <int DH>
struct ChunkPair {
    int j;          // chunk index inside the half head (rotation-table offset 8j)
    int64_t lo, hi; // first channel of the low and the high half
    MAGLEV_DEV explicit ChunkPair(int cp)
    {
        constexpr int PER_HEAD = DH / 16;
        j = cp % PER_HEAD;
        lo = (int64_t)(cp / PER_HEAD) * DH + 8 * j;
        hi = lo + DH / 2;
    }
};

// The workgroup's copy of the gate values g = 2 sigmoid(a), [4][HD] floats in
// LDS (dynamic shared memory, 16 HD bytes): computed once, read per row, so
// that the gates do not occupy 64 registers per thread.
MAGLEV_DEV void stage_gates(const float *logits, int n, float *gsh)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x) gsh[i] = two_sigmoid(logits[i]);
    __syncthreads();
}

MAGLEV_DEV void lds8(const float *p, float *out)
{
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
}

struct GatedArgs {
    int64_t N, Tlen, pos0;
    int HD, rows_per_block;
    int row_threads;      // threads a row takes (a multiple of 64)
    float eps;
    const float2 *rope;   // [pos][Dh/2] or nullptr
    const float *gates;   // [4][HD] logits: a_kl, a_kr, a_vl, a_vr
};

// Eight elements as loaded (bf16 kept packed, converted when used), so that a
// row's loads can all be in flight in few registers.
template <typename T> struct Chunk8;
template <> struct Chunk8<bf16> {
    u32x4 x;
    MAGLEV_DEV void load(const bf16 *p) { x = *reinterpret_cast<const u32x4 *>(p); }
    MAGLEV_DEV void zero() { x = u32x4{0u, 0u, 0u, 0u}; }
    MAGLEV_DEV void get(float *out) const
    {
        const bf16x8 v = __builtin_bit_cast(bf16x8, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
    }
};
template <> struct Chunk8<float> {
    f32x4 a, b;
    MAGLEV_DEV void load(const float *p)
    {
        a = *reinterpret_cast<const f32x4 *>(p);
        b = *reinterpret_cast<const f32x4 *>(p + 4);
    }
    MAGLEV_DEV void zero() { a = b = f32x4{0.f, 0.f, 0.f, 0.f}; }
    MAGLEV_DEV void get(float *out) const
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
    }
};

// ---------------------------------------------------------------------------
// Forward: mixed entries kx, vx from k, v, kp (pre-norm), vm.
// A row's eight loads go out together; two row groups a workgroup keep two
// rows in flight (the row norm's sum is the only step that waits on other
// threads).
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ __launch_bounds__(256) void gated_mix_fwd(GatedArgs a, const T *k, const T *v,
                                                      const T *kp, const T *vm, T *kx, T *vx)
{
    // Row groups as in the backward: nh groups of rt threads, group h taking
    // rows r0 + h, r0 + h + nh, ..., one row in flight each.
    __shared__ float red[2][2][4];   // [iteration parity][group][wave of the group]
    extern __shared__ __attribute__((aligned(16))) float gsh[];   // [4][HD]
    const int rt = a.row_threads, nh = blockDim.x / rt;
    const int tid = threadIdx.x, grp = tid / rt, tig = tid - grp * rt;
    const int nwg = rt >> 6, wig = tig >> 6;
    const bool act = tig < a.HD / 16;
    const ChunkPair<DH> cp(act ? tig : 0);
    const int64_t r0 = (int64_t)blockIdx.x * a.rows_per_block;
    const int64_t r1 = r0 + a.rows_per_block < a.N ? r0 + a.rows_per_block : a.N;
    const int64_t niter = r1 > r0 ? (r1 - r0 + nh - 1) / nh : 0;
    auto row_of = [&](int64_t it) { return r0 + it * nh + grp; };
    // [kp, k, v, vm][low, high half]
    using RowIn = Chunk8<T>[4][2];
    auto load_row = [&](int64_t row, RowIn &d) {
        const int64_t base = row * a.HD;
        const T *src[4] = {kp, k, v, vm};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (act && row < r1) {
                d[t][0].load(src[t] + base + cp.lo);
                d[t][1].load(src[t] + base + cp.hi);
            } else {
                d[t][0].zero();
                d[t][1].zero();
            }
        }
    };
    RowIn ia;
    if (niter > 0) load_row(row_of(0), ia);
    stage_gates(a.gates, 4 * a.HD, gsh);
    const float *gk = gsh, *gv = gsh + 2 * a.HD;   // [2][HD] each: local, recurrent
    const float inv_hd = 1.0f / (float)a.HD;
    auto mix_row = [&](int64_t it, const RowIn &d) {
        const int64_t row = row_of(it);
        const int64_t base = row * a.HD;
        float nl[8], nh[8];
        d[0][0].get(nl);
        d[0][1].get(nh);
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += nl[e] * nl[e] + nh[e] * nh[e];
        const float rs = rsqrtf(group_sum(ss, red[it & 1][grp], nwg, wig) * inv_hd + a.eps);
        if (!act || row >= r1) return;
        float kl[8], kh[8];
        d[1][0].get(kl);
        d[1][1].get(kh);
#pragma unroll
        for (int e = 0; e < 8; ++e) { nl[e] *= rs; nh[e] *= rs; }
        if (a.rope) {
            const float2 *cs = a.rope + (a.pos0 + row % a.Tlen) * (DH / 2) + 8 * cp.j;
            rotate_pairs(kl, kh, cs, false);
            rotate_pairs(nl, nh, cs, false);
        }
        {
            float ga[8], gb[8];
            lds8(gk + cp.lo, ga);
            lds8(gk + a.HD + cp.lo, gb);
#pragma unroll
            for (int e = 0; e < 8; ++e) kl[e] = ga[e] * kl[e] + gb[e] * nl[e];
            lds8(gk + cp.hi, ga);
            lds8(gk + a.HD + cp.hi, gb);
#pragma unroll
            for (int e = 0; e < 8; ++e) kh[e] = ga[e] * kh[e] + gb[e] * nh[e];
        }
        store8(kx + base + cp.lo, kl);
        store8(kx + base + cp.hi, kh);
        float vl[8], vh[8], ml[8], mh[8];
        d[2][0].get(vl);
        d[2][1].get(vh);
        d[3][0].get(ml);
        d[3][1].get(mh);
        {
            float ga[8], gb[8];
            lds8(gv + cp.lo, ga);
            lds8(gv + a.HD + cp.lo, gb);
#pragma unroll
            for (int e = 0; e < 8; ++e) vl[e] = ga[e] * vl[e] + gb[e] * ml[e];
            lds8(gv + cp.hi, ga);
            lds8(gv + a.HD + cp.hi, gb);
#pragma unroll
            for (int e = 0; e < 8; ++e) vh[e] = ga[e] * vh[e] + gb[e] * mh[e];
        }
        store8(vx + base + cp.lo, vl);
        store8(vx + base + cp.hi, vh);
    };
    for (int64_t it = 0; it < niter; ++it) {
        if (it > 0) load_row(row_of(it), ia);
        mix_row(it, ia);
    }
}

// ---------------------------------------------------------------------------
// Backward. dk/dv hold dk~/dv~ on entry and dk/dv on exit (each thread reads
// its channels before it overwrites them). dkp, dvm receive the gradients of
// the projected memory; gpart[block][4][HD] the per-block gate partial sums
// (before the 2 sigma (1 - sigma) factor).
// dkn = R^T (g_kr (.) dk~) does not depend on the norm, and
// mean(dkn (.) kn) = rs * mean(dkn (.) kp) with rs = 1/rms, so both row sums
// (of kp^2 and of dkn (.) kp) come out of one reduction. A row's twelve loads
// go out together.
// ---------------------------------------------------------------------------
// Sums of x and y over the nw waves of one row group (red: one slot per wave
// of the group, wave index wi inside it); every thread of the workgroup must
// call it, since it holds the workgroup barrier.
MAGLEV_DEV float2 group_sum2(float x, float y, float2 *red, int nw, int wi)
{
    x = wave_sum(x);
    y = wave_sum(y);
    if ((threadIdx.x & 63) == 0) red[wi] = make_float2(x, y);
    __syncthreads();
    float2 t = make_float2(0.0f, 0.0f);
    for (int i = 0; i < nw; ++i) { t.x += red[i].x; t.y += red[i].y; }
    return t;
}

// Eight projection gradients into dkp/dvm: rounded to the storage type, or
// (float32 targets of a stack sharing one projection) written or added.
MAGLEV_DEV void put8(bf16 *p, const float *in, bool) { store8(p, in); }
MAGLEV_DEV void put8(float *p, const float *in, bool add)
{
    if (!add) { store8(p, in); return; }
    f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] += in[i]; b[i] += in[4 + i]; }
    *reinterpret_cast<f32x4 *>(p) = a;
    *reinterpret_cast<f32x4 *>(p + 4) = b;
}

// PT: type of the projection gradients dkp, dvm (T, or float32 sums over the
// layers of a shared projection; padd: add to them).
template <typename T, int DH, typename PT>
__global__ __launch_bounds__(256, 2) void gated_mix_bwd(GatedArgs a, const T *k, const T *v,
                                                      const T *kp, const T *vm, T *dk, T *dv,
                                                      PT *dkp, PT *dvm, bool padd, float *gpart)
{
    // The workgroup is nh row groups of rt threads (nh = 2 when a row needs at
    // most 128 threads): group h takes rows r0 + h, r0 + h + nh, ..., so that
    // two waves a SIMD work while the per-block gate partials stay as few as
    // with one group. Both groups run the same number of iterations (a group
    // past the block's last row runs one without loads or stores), since the
    // row reductions hold workgroup barriers.
    __shared__ float2 red[2][2][4];   // [iteration parity][group][wave of the group]
    extern __shared__ __attribute__((aligned(16))) float gsh[];   // [4][HD] gates, [64][rt] partials
    const int rt = a.row_threads, nh = blockDim.x / rt;
    const int tid = threadIdx.x, grp = tid / rt, tig = tid - grp * rt;
    const int nwg = rt >> 6, wig = tig >> 6;
    const bool act = tig < a.HD / 16;
    const ChunkPair<DH> cp(act ? tig : 0);
    const int64_t r0 = (int64_t)blockIdx.x * a.rows_per_block;
    const int64_t r1 = r0 + a.rows_per_block < a.N ? r0 + a.rows_per_block : a.N;
    const int64_t niter = r1 > r0 ? (r1 - r0 + nh - 1) / nh : 0;
    auto row_of = [&](int64_t it) { return r0 + it * nh + grp; };
    // [kp, dk~, k, dv~, v, vm][low, high half]
    using RowIn = Chunk8<T>[6][2];
    auto load_row = [&](int64_t row, RowIn &d) {
        const int64_t base = row * a.HD;
        const T *src[6] = {kp, dk, k, dv, v, vm};
#pragma unroll
        for (int t = 0; t < 6; ++t) {
            if (act && row < r1) {
                d[t][0].load(src[t] + base + cp.lo);
                d[t][1].load(src[t] + base + cp.hi);
            } else {
                d[t][0].zero();
                d[t][1].zero();
            }
        }
    };
    RowIn ia;
    if (niter > 0) load_row(row_of(0), ia);
    stage_gates(a.gates, 4 * a.HD, gsh);
    const float *gkl = gsh, *gkr = gsh + a.HD, *gvl = gsh + 2 * a.HD, *gvr = gsh + 3 * a.HD;
    float pkl[16] = {}, pkr[16] = {}, pvl[16] = {}, pvr[16] = {};
    const float inv_hd = 1.0f / (float)a.HD;
    auto grad_row = [&](int64_t it, const RowIn &d) {
        const int64_t row = row_of(it);
        const bool live = act && row < r1;
        const int64_t base = row * a.HD;
        const float2 *cs = (live && a.rope) ? a.rope + (a.pos0 + row % a.Tlen) * (DH / 2) + 8 * cp.j
                                            : nullptr;
        float nl[8], nh[8], gl[8], gh[8], dnl[8], dnh[8];
        d[0][0].get(nl);
        d[0][1].get(nh);
        d[1][0].get(gl);
        d[1][1].get(gh);
        {
            float gc[8], gd[8];
            lds8(gkr + cp.lo, gc);
            lds8(gkr + cp.hi, gd);
#pragma unroll
            for (int e = 0; e < 8; ++e) { dnl[e] = gc[e] * gl[e]; dnh[e] = gd[e] * gh[e]; }
        }
        if (cs) rotate_pairs(dnl, dnh, cs, true);   // dkn
        float ss = 0.0f, sd = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ss += nl[e] * nl[e] + nh[e] * nh[e];
            sd += dnl[e] * nl[e] + dnh[e] * nh[e];
        }
        const float2 t = group_sum2(ss, sd, red[it & 1][grp], nwg, wig);
        const float rs = rsqrtf(t.x * inv_hd + a.eps);
        const float mu = t.y * rs * inv_hd;   // mean(dkn (.) kn)
        if (!live) return;
#pragma unroll
        for (int e = 0; e < 8; ++e) { nl[e] *= rs; nh[e] *= rs; }   // kn
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            dnl[e] = (dnl[e] - nl[e] * mu) * rs;
            dnh[e] = (dnh[e] - nh[e] * mu) * rs;
        }
        put8(dkp + base + cp.lo, dnl, padd);
        put8(dkp + base + cp.hi, dnh, padd);
        float kl[8], kh[8];
        d[2][0].get(kl);
        d[2][1].get(kh);
        if (cs) {
            rotate_pairs(kl, kh, cs, false);
            rotate_pairs(nl, nh, cs, false);
        }
        float ol[8], oh[8];
        {
            float ga[8], gb[8];
            lds8(gkl + cp.lo, ga);
            lds8(gkl + cp.hi, gb);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pkl[e] += gl[e] * kl[e];
                pkl[8 + e] += gh[e] * kh[e];
                pkr[e] += gl[e] * nl[e];
                pkr[8 + e] += gh[e] * nh[e];
                ol[e] = ga[e] * gl[e];
                oh[e] = gb[e] * gh[e];
            }
        }
        if (cs) rotate_pairs(ol, oh, cs, true);
        store8(dk + base + cp.lo, ol);
        store8(dk + base + cp.hi, oh);

        float vl[8], vh[8], ml[8], mh[8];
        d[3][0].get(gl);
        d[3][1].get(gh);
        d[4][0].get(vl);
        d[4][1].get(vh);
        d[5][0].get(ml);
        d[5][1].get(mh);
        {
            float ga[8], gb[8], gc[8], gd[8];
            lds8(gvl + cp.lo, ga);
            lds8(gvl + cp.hi, gb);
            lds8(gvr + cp.lo, gc);
            lds8(gvr + cp.hi, gd);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pvl[e] += gl[e] * vl[e];
                pvl[8 + e] += gh[e] * vh[e];
                pvr[e] += gl[e] * ml[e];
                pvr[8 + e] += gh[e] * mh[e];
                vl[e] = ga[e] * gl[e];
                vh[e] = gb[e] * gh[e];
                ml[e] = gc[e] * gl[e];
                mh[e] = gd[e] * gh[e];
            }
        }
        store8(dv + base + cp.lo, vl);
        store8(dv + base + cp.hi, vh);
        put8(dvm + base + cp.lo, ml, padd);
        put8(dvm + base + cp.hi, mh, padd);
    };
    // One row in flight per group: the second group is what overlaps a row's
    // loads with another's reduction (a prefetched row per group costs the
    // registers of two waves a SIMD: 107 µs at d20 against 139 µs).
    for (int64_t it = 0; it < niter; ++it) {
        if (it > 0) load_row(row_of(it), ia);
        grad_row(it, ia);
    }
    float *parts[4] = {pkl, pkr, pvl, pvr};
    if (nh > 1) {
        // group 1 hands its partial sums to group 0 through LDS ([64][rt]
        // after the gates), which adds them in a fixed order
        float *pp = gsh + 4 * a.HD;
        if (grp == 1 && act) {
#pragma unroll
            for (int gi = 0; gi < 4; ++gi)
#pragma unroll
                for (int e = 0; e < 16; ++e) pp[(gi * 16 + e) * rt + tig] = parts[gi][e];
        }
        __syncthreads();
        if (grp == 0 && act) {
#pragma unroll
            for (int gi = 0; gi < 4; ++gi)
#pragma unroll
                for (int e = 0; e < 16; ++e) parts[gi][e] += pp[(gi * 16 + e) * rt + tig];
        }
    }
    if (grp != 0 || !act) return;
    float *out = gpart + (int64_t)blockIdx.x * 4 * a.HD;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
        store8(out + gi * a.HD + cp.lo, parts[gi]);
        store8(out + gi * a.HD + cp.hi, parts[gi] + 8);
    }
}

// dgates[i] (+)= 2 sigmoid(a_i)(1 - sigmoid(a_i)) * sum_b gpart[b][i], the
// blocks summed in a fixed order. One wave per 64 outputs and per quarter of
// the blocks; the quarters are combined in order through LDS.
__global__ __launch_bounds__(256) void gate_grad_reduce(const float *gpart, int nblk, int n,
                                                        const float *gates, float *dgates,
                                                        unsigned acc)
{
    __shared__ float part[4][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i = blockIdx.x * 64 + lane;
    float s = 0.0f;
    if (i < n) {
        const int per = (nblk + 3) / 4;
        const int b0 = w * per, b1 = b0 + per < nblk ? b0 + per : nblk;
#pragma unroll 8
        for (int b = b0; b < b1; ++b) s += gpart[(int64_t)b * n + i];
    }
    part[w][lane] = s;
    __syncthreads();
    if (w == 0 && i < n) {
        const float tot = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
        const float sg = 1.0f / (1.0f + __expf(-gates[i]));
        const float g = 2.0f * sg * (1.0f - sg) * tot;
        dgates[i] = acc ? dgates[i] + g : g;
    }
}

unsigned row_threads(int HD) { return (unsigned)((HD / 16 + 63) / 64 * 64); }
size_t gate_lds_bytes(int HD) { return (size_t)4 * HD * sizeof(float); }

GatedArgs gated_args(const Geom &g, const float *gates, float eps, const float2 *rope,
                     int rows_per_block)
{
    GatedArgs a;
    a.N = g.N(); a.Tlen = g.T; a.pos0 = g.pos0;
    a.HD = g.HD(); a.rows_per_block = rows_per_block;
    a.row_threads = (int)row_threads(g.HD());
    a.eps = eps; a.rope = rope; a.gates = gates;
    return a;
}

template <typename T, int DH>
void fwd_t(const Geom &g, const void *k, const void *v, const void *kp, const void *vm,
           const float *gates, float eps, const float2 *rope, void *kx, void *vx, hipStream_t s)
{
    const int rpb = kGatedFwdRows;
    const GatedArgs a = gated_args(g, gates, eps, rope, rpb);
    const unsigned nblk = (unsigned)((g.N() + rpb - 1) / rpb);
    const unsigned rt = row_threads(g.HD()), nh = rt <= 128 ? 2u : 1u;
    prof::Scope ts("gated_mix", s);
    hipLaunchKernelGGL((gated_mix_fwd<T, DH>), dim3(nblk), dim3(nh * rt), gate_lds_bytes(g.HD()), s, a,
                       static_cast<const T *>(k), static_cast<const T *>(v),
                       static_cast<const T *>(kp), static_cast<const T *>(vm),
                       static_cast<T *>(kx), static_cast<T *>(vx));
}

template <typename T, int DH, typename PT>
void bwd_t(const Geom &g, const void *k, const void *v, const void *kp, const void *vm,
           const float *gates, float eps, const float2 *rope, void *dk, void *dv, PT *dkp,
           PT *dvm, bool padd, const BwdWorkspace &ws, float *dgates, unsigned acc, hipStream_t s)
{
    const GatedArgs a = gated_args(g, gates, eps, rope, ws.g_rows);
    {
        // two row groups a workgroup when a row takes at most 128 threads
        const unsigned rt = row_threads(g.HD()), nh = rt <= 128 ? 2u : 1u;
        const size_t lds = gate_lds_bytes(g.HD()) + (nh > 1 ? (size_t)64 * rt * sizeof(float) : 0);
        prof::Scope ts("gated_mix_bwd", s);
        hipLaunchKernelGGL((gated_mix_bwd<T, DH, PT>), dim3((unsigned)ws.g_blocks), dim3(nh * rt),
                           lds, s, a, static_cast<const T *>(k), static_cast<const T *>(v),
                           static_cast<const T *>(kp), static_cast<const T *>(vm),
                           static_cast<T *>(dk), static_cast<T *>(dv), dkp, dvm, padd, ws.gpart);
    }
    const int n = 4 * g.HD();
    prof::Scope ts("gate_grad_reduce", s);
    hipLaunchKernelGGL(gate_grad_reduce, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, s, ws.gpart,
                       ws.g_blocks, n, gates, dgates, (acc & 4u) != 0u);
}

}  // namespace

void gated_partition(int64_t N, int *rows_per_block, int *blocks)
{
    // About 512 workgroups (two per CU), at least 8 rows each so that the
    // per-block gate partials stay small next to the activations.
    int64_t rpb = (N + 511) / 512;
    if (rpb < 8) rpb = 8;
    int64_t nb = (N + rpb - 1) / rpb;
    if (nb < 1) nb = 1;
    *rows_per_block = (int)rpb;
    *blocks = (int)nb;
}

hipError_t launch_gated_mix(const Geom &g, const void *k, const void *v, const void *kp,
                            const void *vm, const float *gates, float eps, const float2 *rope,
                            void *kx, void *vx, hipStream_t s)
{
    if (g.dtype == MAGLEV_BF16) {
        if (g.Dh == 128) fwd_t<bf16, 128>(g, k, v, kp, vm, gates, eps, rope, kx, vx, s);
        else fwd_t<bf16, 64>(g, k, v, kp, vm, gates, eps, rope, kx, vx, s);
    } else {
        if (g.Dh == 128) fwd_t<float, 128>(g, k, v, kp, vm, gates, eps, rope, kx, vx, s);
        else fwd_t<float, 64>(g, k, v, kp, vm, gates, eps, rope, kx, vx, s);
    }
    return hipGetLastError();
}

hipError_t launch_gated_mix_bwd(const Geom &g, const void *k, const void *v, const void *kp,
                                const void *vm, const float *gates, float eps,
                                const float2 *rope, void *dk, void *dv, const BwdWorkspace &ws,
                                float *dgates, unsigned acc, float *dkp32, float *dvm32,
                                hipStream_t s)
{
    const bool f32 = dkp32 != nullptr, padd = f32 && (acc & 1u);
#define MAGLEV_GATED_BWD(T, DH)                                                               \
    (f32 ? bwd_t<T, DH, float>(g, k, v, kp, vm, gates, eps, rope, dk, dv, dkp32, dvm32, padd,  \
                               ws, dgates, acc, s)                                            \
         : bwd_t<T, DH, T>(g, k, v, kp, vm, gates, eps, rope, dk, dv, static_cast<T *>(ws.dkp), \
                           static_cast<T *>(ws.dvm), false, ws, dgates, acc, s))
    if (g.dtype == MAGLEV_BF16) {
        if (g.Dh == 128) MAGLEV_GATED_BWD(bf16, 128);
        else MAGLEV_GATED_BWD(bf16, 64);
    } else {
        if (g.Dh == 128) MAGLEV_GATED_BWD(float, 128);
        else MAGLEV_GATED_BWD(float, 64);
    }
#undef MAGLEV_GATED_BWD
    return hipGetLastError();
}

}  // namespace maglev
