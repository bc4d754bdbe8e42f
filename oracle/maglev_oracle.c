/*
 * maglev_oracle.c -- plain, slow, double-precision CPU oracle for the Maglev
 * decoder-P attention path with recurrent K/V injection.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header, table or
 * constant with the HIP library, and the HIP library never calls it.
 *
 * Sources (web summaries of the preprint "Maglev: Sliding Recurrent Memory"):
 *   [R-bg]   paper.rainbus.top, "Maglev：滑动窗口循环记忆", section 前置知识
 *            (background: sliding-window attention keeps the W most recent
 *            tokens; the KV cache; the feature-consistency loss; RoPE rotates
 *            q and k by an angle set by absolute position so that scores depend
 *            only on the offset, and both the local and the injected key are
 *            rotated before they are mixed).
 *   [R-mot]  same page, section 研究动机 (the interface
 *            p(x_{t+1}, m_t | x_{t-W+1:t}, M_{t-1}) with a W-entry memory window).
 *   [R-core] same page, section 核心方法 (P is all sliding-window, W = 512;
 *            shifted memory enters through a shared projection into K/V
 *            features mixed into the existing cache entries; loss term
 *            lambda*||m_t - m'_t||^2 / sqrt(d)).
 *   [R-step] same page, section 方法步骤详情 (P consumes m'_{0:T-1} with
 *            m'_0 = 0; recurrent K/V features from W^rec m'_{t-1}; gated mix
 *            with the local features; attention over the W most recent mixed
 *            entries; loss averaged over positions; recurrent inference).
 *   [G-inf]  gist.science, "Technische Samenvatting: Maglev - Sliding Recurrent
 *            Memory", section Inferentiemechanisme (memory rides in the K/V
 *            cache; bounded cost).
 *
 * Mixing form. The pages print one summary's gated variant but leave the exact
 * form open; this oracle implements the form the library fixes:
 *     k~_j = R_j k_j + s_h * R_j (W_Km m'_{j-1}),   v~_j = v_j + s_h * W_Vm m'_{j-1},
 *     s_h  = 1 / (1 + exp(-g_h)), one gate logit per head.
 * The gated variant that [R-step] prints (channel-wise 2*sigma gates on both
 * terms, RMSNorm on the projected memory key) follows at the end of the file.
 *
 * Conventions where the pages are silent (each listed with its reading in the
 * design notes): RoPE pairs channel i with i + Dh/2, theta_i = base^(-2i/Dh),
 * angle = position * theta_i, positions pos0 + t; V is not rotated; the window
 * holds exactly W keys including the query's own position (0 <= i - j <= W-1);
 * softmax scale 1/sqrt(Dh) unless given; masked pairs are excluded, not
 * penalised; the loss divides the squared L2 norm by sqrt(d) and averages over
 * all N = B*T positions.
 *
 * Everything is double precision. Inputs arrive as doubles holding exactly the
 * stored values (bf16 or fp32). Layouts, row-major:
 *   q,k,v,kmem,vmem,o,dO,dq,dk,dv [B,T,H,Dh]; m, m' [B,T,d];
 *   W_Km, W_Vm [H*Dh, d]; lse [B,H,T]; ring caches [Bs,H,W,Dh].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* Gate nonlinearity s = sigma(g). g = -inf gives exactly 0, g = +inf exactly 1. */
static double gate_sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }

/* Rotate x[0..Dh) by the RoPE angle of absolute position p ([R-bg]).
 * Channel i pairs with channel i + Dh/2; inverse != 0 applies R^T.
 * base <= 0 disables the rotation. */
static void rope_rotate(double *x, int Dh, double p, double base, int inverse)
{
    if (base <= 0.0) return;
    const int half = Dh / 2;
    for (int i = 0; i < half; ++i) {
        const double theta = pow(base, -2.0 * (double)i / (double)Dh);
        const double phi = p * theta;
        const double c = cos(phi);
        const double s = inverse ? -sin(phi) : sin(phi);
        const double a = x[i], b = x[i + half];
        x[i] = a * c - b * s;
        x[i + half] = a * s + b * c;
    }
}

static double dot(const double *a, const double *b, int n)
{
    double acc = 0.0;
    for (int i = 0; i < n; ++i) acc += a[i] * b[i];
    return acc;
}

/* Round a double to the nearest bfloat16 value, ties to even, keeping it as a
 * double. Used only where the data structure itself stores bf16 (the decode
 * ring cache holds bf16 entries). */
ORACLE_API double oracle_round_bf16(double x)
{
    if (!isfinite(x) || x == 0.0) return x;
    int e;
    (void)frexp(x, &e);              /* x = f * 2^e with 0.5 <= |f| < 1 */
    int qexp = e - 8;                /* 8 significant bits */
    if (qexp < -133) qexp = -133;    /* bf16 subnormal quantum */
    const double quantum = ldexp(1.0, qexp);
    double r = nearbyint(x / quantum) * quantum;   /* default mode: ties to even */
    const double maxv = ldexp(255.0, 120);          /* (2 - 2^-7) * 2^127 */
    if (r > maxv) r = INFINITY;
    if (r < -maxv) r = -INFINITY;
    return r;
}

/* ---------------------------------------------------------------------------
 * Shift and memory projection ([R-step]): P consumes m'_{0:T-1} with m'_0 = 0,
 * i.e. row t of the projection input is m'[t-1] and row 0 is zero when
 * shift = 1; shift = 0 uses m[t] itself (the decode step injects m_{t-1}
 * directly). kmem = W_Km * input, vmem = W_Vm * input, split per head.
 * ------------------------------------------------------------------------- */
ORACLE_API void oracle_mem_project(int64_t B, int64_t T, int H, int Dh, int d, int shift,
                                   const double *m, const double *W_Km, const double *W_Vm,
                                   double *kmem, double *vmem)
{
    const int HD = H * Dh;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t t = 0; t < T; ++t) {
            const int64_t src_t = t - shift;
            const double *src = (src_t >= 0) ? m + (b * T + src_t) * d : NULL;
            double *ko = kmem + (b * T + t) * HD;
            double *vo = vmem + (b * T + t) * HD;
            for (int r = 0; r < HD; ++r) {
                ko[r] = src ? dot(W_Km + (int64_t)r * d, src, d) : 0.0;
                vo[r] = src ? dot(W_Vm + (int64_t)r * d, src, d) : 0.0;
            }
        }
    }
}

/* Rotated query, mixed key and mixed value of one (b, h) sequence, plus the
 * rotated memory key (kept for the gate derivative). */
typedef struct {
    double *qh, *kt, *vt, *rk;   /* each [T][Dh] */
} head_view;

static int head_view_alloc(head_view *hv, int64_t T, int Dh)
{
    const size_t n = (size_t)T * (size_t)Dh;
    hv->qh = malloc(n * sizeof(double));
    hv->kt = malloc(n * sizeof(double));
    hv->vt = malloc(n * sizeof(double));
    hv->rk = malloc(n * sizeof(double));
    return hv->qh && hv->kt && hv->vt && hv->rk;
}

static void head_view_free(head_view *hv)
{
    free(hv->qh); free(hv->kt); free(hv->vt); free(hv->rk);
}

/* Build q^ = R q, k~ = R k + s R kmem, v~ = v + s vmem for sequence (b, h). */
static void head_view_fill(head_view *hv, int64_t b, int h, int64_t T, int H, int Dh,
                           int64_t pos0, double base, double s,
                           const double *q, const double *k, const double *v,
                           const double *kmem, const double *vmem)
{
    for (int64_t t = 0; t < T; ++t) {
        const int64_t off = ((b * T + t) * H + h) * Dh;
        const double p = (double)(pos0 + t);
        double *qh = hv->qh + t * Dh, *kt = hv->kt + t * Dh;
        double *vt = hv->vt + t * Dh, *rk = hv->rk + t * Dh;
        memcpy(qh, q + off, (size_t)Dh * sizeof(double));
        rope_rotate(qh, Dh, p, base, 0);
        memcpy(kt, k + off, (size_t)Dh * sizeof(double));
        rope_rotate(kt, Dh, p, base, 0);
        memcpy(rk, kmem + off, (size_t)Dh * sizeof(double));
        rope_rotate(rk, Dh, p, base, 0);
        for (int c = 0; c < Dh; ++c) {
            kt[c] = kt[c] + s * rk[c];
            vt[c] = v[off + c] + s * vmem[off + c];
        }
    }
}

/* Mixed cache entries of every position ([R-bg]: both the local key and the
 * injected memory key are rotated before they are mixed; [R-step]: the gated
 * mix with the local K/V features):
 *     kmix_t = R_t k_t + s_h R_t kmem_t,   vmix_t = v_t + s_h vmem_t,
 * with R_t the rotation of absolute position pos0 + t. */
ORACLE_API void oracle_mixed_entries(int64_t B, int64_t T, int H, int Dh, int64_t pos0,
                                     double base, const double *k, const double *v,
                                     const double *kmem, const double *vmem,
                                     const double *gate_logit, double *kmix, double *vmix)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t t = 0; t < T; ++t) {
            double rk[512], rm[512];
            const double p = (double)(pos0 + t);
            for (int h = 0; h < H; ++h) {
                const int64_t off = ((b * T + t) * H + h) * Dh;
                const double s = gate_sigmoid(gate_logit[h]);
                memcpy(rk, k + off, (size_t)Dh * sizeof(double));
                rope_rotate(rk, Dh, p, base, 0);
                memcpy(rm, kmem + off, (size_t)Dh * sizeof(double));
                rope_rotate(rm, Dh, p, base, 0);
                for (int c = 0; c < Dh; ++c) {
                    kmix[off + c] = rk[c] + s * rm[c];
                    vmix[off + c] = v[off + c] + s * vmem[off + c];
                }
            }
        }
    }
}

static double default_scale(double scale, int Dh) { return scale > 0.0 ? scale : 1.0 / sqrt((double)Dh); }

/* Softmax weights of query i over its window J(i) = {max(0, i-W+1) .. i}
 * ([R-bg], [R-step]). p[j - lo] receives P_ij; returns lo; *lse_out = ln sum exp S. */
static int64_t window_softmax(const head_view *hv, int64_t i, int64_t W, int Dh, double scale,
                              double *p, double *lse_out)
{
    const int64_t lo = (i - W + 1) > 0 ? (i - W + 1) : 0;
    const double *qi = hv->qh + i * Dh;
    double mx = -INFINITY;
    for (int64_t j = lo; j <= i; ++j) {
        p[j - lo] = scale * dot(qi, hv->kt + j * Dh, Dh);
        if (p[j - lo] > mx) mx = p[j - lo];
    }
    double sum = 0.0;
    for (int64_t j = lo; j <= i; ++j) {
        p[j - lo] = exp(p[j - lo] - mx);
        sum += p[j - lo];
    }
    for (int64_t j = lo; j <= i; ++j) p[j - lo] /= sum;
    if (lse_out) *lse_out = mx + log(sum);
    return lo;
}

/* ---------------------------------------------------------------------------
 * Forward: sliding-window attention over the W most recent mixed entries.
 * o [B,T,H,Dh]; lse [B,H,T] (may be NULL).
 * ------------------------------------------------------------------------- */
ORACLE_API void oracle_swa_inject_fwd(int64_t B, int64_t T, int H, int Dh, int64_t W,
                                      int64_t pos0, double rope_base, double scale,
                                      const double *q, const double *k, const double *v,
                                      const double *kmem, const double *vmem,
                                      const double *gate_logit, double *o, double *lse)
{
    scale = default_scale(scale, Dh);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            head_view hv;
            double *p = malloc((size_t)(W < T ? W : T) * sizeof(double));
            if (!head_view_alloc(&hv, T, Dh) || !p) abort();
            const double s = gate_sigmoid(gate_logit[h]);
            head_view_fill(&hv, b, h, T, H, Dh, pos0, rope_base, s, q, k, v, kmem, vmem);
            for (int64_t i = 0; i < T; ++i) {
                double l;
                const int64_t lo = window_softmax(&hv, i, W, Dh, scale, p, &l);
                double *oi = o + ((b * T + i) * H + h) * Dh;
                for (int c = 0; c < Dh; ++c) oi[c] = 0.0;
                for (int64_t j = lo; j <= i; ++j)
                    for (int c = 0; c < Dh; ++c) oi[c] += p[j - lo] * hv.vt[j * Dh + c];
                if (lse) lse[((int64_t)b * H + h) * T + i] = l;
            }
            free(p);
            head_view_free(&hv);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Backward of the whole layer path, by the chain rule applied to the forward
 * above (plus the shift and projection):
 *   inputs  q, k, v, m', W_Km, W_Vm, gate logits; upstream gradient dO
 *   outputs dq, dk, dv [B,T,H,Dh]; dm' [B,T,d]; dW_Km, dW_Vm [H*Dh,d]; dgate [H]
 * dm' row T-1 receives no injection gradient (m'_T is never consumed).
 * ------------------------------------------------------------------------- */
ORACLE_API void oracle_swa_inject_bwd(int64_t B, int64_t T, int H, int Dh, int d, int64_t W,
                                      int64_t pos0, double rope_base, double scale,
                                      const double *q, const double *k, const double *v,
                                      const double *m_prime, const double *W_Km,
                                      const double *W_Vm, const double *gate_logit,
                                      const double *dO, double *dq, double *dk, double *dv,
                                      double *dm_prime, double *dW_Km, double *dW_Vm,
                                      double *dgate)
{
    scale = default_scale(scale, Dh);
    const int HD = H * Dh;
    const size_t nact = (size_t)B * (size_t)T * (size_t)HD;
    double *kmem = malloc(nact * sizeof(double));
    double *vmem = malloc(nact * sizeof(double));
    double *dkmem = malloc(nact * sizeof(double));   /* d loss / d kmem */
    double *dvmem = malloc(nact * sizeof(double));
    double *ds_bh = calloc((size_t)B * H, sizeof(double));  /* d loss / d s, per (b,h) */
    if (!kmem || !vmem || !dkmem || !dvmem || !ds_bh) abort();

    oracle_mem_project(B, T, H, Dh, d, 1, m_prime, W_Km, W_Vm, kmem, vmem);

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            head_view hv;
            const int64_t wmax = W < T ? W : T;
            double *p = malloc((size_t)wmax * sizeof(double));
            double *dp = malloc((size_t)wmax * sizeof(double));
            double *dqh = calloc((size_t)T * Dh, sizeof(double));   /* d / d q^ */
            double *dkt = calloc((size_t)T * Dh, sizeof(double));   /* d / d k~ */
            double *dvt = calloc((size_t)T * Dh, sizeof(double));   /* d / d v~ */
            double *tmp = malloc((size_t)Dh * sizeof(double));
            if (!head_view_alloc(&hv, T, Dh) || !p || !dp || !dqh || !dkt || !dvt || !tmp) abort();
            const double s = gate_sigmoid(gate_logit[h]);
            head_view_fill(&hv, b, h, T, H, Dh, pos0, rope_base, s, q, k, v, kmem, vmem);

            for (int64_t i = 0; i < T; ++i) {
                const int64_t lo = window_softmax(&hv, i, W, Dh, scale, p, NULL);
                const double *dOi = dO + ((b * T + i) * H + h) * Dh;
                /* dP_ij = <dO_i, v~_j>;  D_i = sum_j P_ij dP_ij */
                double Di = 0.0;
                for (int64_t j = lo; j <= i; ++j) {
                    dp[j - lo] = dot(dOi, hv.vt + j * Dh, Dh);
                    Di += p[j - lo] * dp[j - lo];
                }
                for (int64_t j = lo; j <= i; ++j) {
                    const double pij = p[j - lo];
                    const double dsij = pij * (dp[j - lo] - Di);   /* dS_ij */
                    for (int c = 0; c < Dh; ++c) {
                        dqh[i * Dh + c] += scale * dsij * hv.kt[j * Dh + c];
                        dkt[j * Dh + c] += scale * dsij * hv.qh[i * Dh + c];
                        dvt[j * Dh + c] += pij * dOi[c];
                    }
                }
            }
            double ds = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t off = ((b * T + t) * H + h) * Dh;
                const double pos = (double)(pos0 + t);
                /* q^ = R q  =>  dq = R^T dq^ */
                memcpy(tmp, dqh + t * Dh, (size_t)Dh * sizeof(double));
                rope_rotate(tmp, Dh, pos, rope_base, 1);
                memcpy(dq + off, tmp, (size_t)Dh * sizeof(double));
                /* k~ = R k + s R kmem  =>  dk = R^T dk~, dkmem = s R^T dk~,
                 * d/ds += <R kmem, dk~> */
                memcpy(tmp, dkt + t * Dh, (size_t)Dh * sizeof(double));
                rope_rotate(tmp, Dh, pos, rope_base, 1);
                for (int c = 0; c < Dh; ++c) {
                    dk[off + c] = tmp[c];
                    dkmem[off + c] = s * tmp[c];
                }
                ds += dot(hv.rk + t * Dh, dkt + t * Dh, Dh);
                /* v~ = v + s vmem  =>  dv = dv~, dvmem = s dv~, d/ds += <vmem, dv~> */
                for (int c = 0; c < Dh; ++c) {
                    dv[off + c] = dvt[t * Dh + c];
                    dvmem[off + c] = s * dvt[t * Dh + c];
                }
                ds += dot(vmem + off, dvt + t * Dh, Dh);
            }
            ds_bh[b * H + h] = ds;
            free(p); free(dp); free(dqh); free(dkt); free(dvt); free(tmp);
            head_view_free(&hv);
        }
    }

    /* gate: s = sigma(g)  =>  dg = s (1 - s) d/ds, summed over the batch */
    for (int h = 0; h < H; ++h) {
        const double s = gate_sigmoid(gate_logit[h]);
        double acc = 0.0;
        for (int64_t b = 0; b < B; ++b) acc += ds_bh[b * H + h];
        dgate[h] = s * (1.0 - s) * acc;
    }

    /* projection input row (b,t) is m'[b,t-1] (zero at t = 0):
     *   d/d input[b,t,e] = sum_r dkmem[b,t,r] W_Km[r,e] + dvmem[b,t,r] W_Vm[r,e]
     *   dm'[b,t] = d/d input[b,t+1]  (t <= T-2);  dm'[b,T-1] = 0 */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t t = 0; t < T; ++t) {
            double *out = dm_prime + (b * T + t) * d;
            if (t == T - 1) {
                for (int e = 0; e < d; ++e) out[e] = 0.0;
                continue;
            }
            const double *gk = dkmem + (b * T + t + 1) * HD;
            const double *gv = dvmem + (b * T + t + 1) * HD;
            for (int e = 0; e < d; ++e) {
                double acc = 0.0;
                for (int r = 0; r < HD; ++r)
                    acc += gk[r] * W_Km[(int64_t)r * d + e] + gv[r] * W_Vm[(int64_t)r * d + e];
                out[e] = acc;
            }
        }
    }

    /*   dW_Km[r,e] = sum_{b,t} dkmem[b,t,r] * input[b,t,e]   (dW_Vm likewise) */
#pragma omp parallel for schedule(static)
    for (int r = 0; r < HD; ++r) {
        for (int e = 0; e < d; ++e) {
            double ak = 0.0, av = 0.0;
            for (int64_t b = 0; b < B; ++b) {
                for (int64_t t = 1; t < T; ++t) {
                    const double x = m_prime[(b * T + t - 1) * d + e];
                    ak += dkmem[(b * T + t) * HD + r] * x;
                    av += dvmem[(b * T + t) * HD + r] * x;
                }
            }
            dW_Km[(int64_t)r * d + e] = ak;
            dW_Vm[(int64_t)r * d + e] = av;
        }
    }
    free(kmem); free(vmem); free(dkmem); free(dvmem); free(ds_bh);
}

/* ---------------------------------------------------------------------------
 * Memory-consistency loss ([R-core], [R-step]):
 *   L = lambda / (N sqrt(d)) * sum_{n,e} (m - m')^2,  dm = 2 lambda (m - m') / (N sqrt(d)),
 *   dm' = -dm.  dm / dm_prime may be NULL.  Returns L.
 * ------------------------------------------------------------------------- */
ORACLE_API double oracle_consistency_loss(int64_t N, int d, double lambda, const double *m,
                                          const double *m_prime, double *dm, double *dm_prime)
{
    const double c = lambda / ((double)N * sqrt((double)d));
    double acc = 0.0;
    for (int64_t i = 0; i < N * (int64_t)d; ++i) {
        const double diff = m[i] - m_prime[i];
        acc += diff * diff;
        if (dm) dm[i] = 2.0 * c * diff;
        if (dm_prime) dm_prime[i] = -2.0 * c * diff;
    }
    return c * acc;
}

/* ---------------------------------------------------------------------------
 * One recurrent decode step ([R-step], [R-mot], [G-inf]) on a W-slot ring.
 * Stream b is at absolute position pos[b]; its new mixed entry
 *   k~ = R_p k + s R_p kmem,  v~ = v + s vmem   (kmem/vmem project m_{t-1})
 * is written to slot pos mod W (rounded to bf16 when ring_bf16 != 0, since the
 * cache then stores bf16). Slot s' holds position p - ((p - s') mod W) and is
 * valid iff that position is >= 0. The rotated query attends over the valid
 * slots. q,k,v,kmem,vmem,o [Bs,H,Dh]; caches [Bs,H,W,Dh] (in/out).
 * ------------------------------------------------------------------------- */
ORACLE_API void oracle_decode_step(int64_t Bs, int H, int Dh, int64_t W, double rope_base,
                                   double scale, int ring_bf16,
                                   const double *q, const double *k, const double *v,
                                   const double *kmem, const double *vmem,
                                   const double *gate_logit, double *kcache, double *vcache,
                                   const int64_t *pos, double *o)
{
    scale = default_scale(scale, Dh);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < Bs; ++b) {
        for (int h = 0; h < H; ++h) {
            double *qh = malloc((size_t)Dh * sizeof(double));
            double *rkl = malloc((size_t)Dh * sizeof(double));
            double *rk = malloc((size_t)Dh * sizeof(double));
            double *sc = malloc((size_t)W * sizeof(double));
            if (!qh || !rkl || !rk || !sc) abort();
            const int64_t p = pos[b];
            const int64_t slot = p % W;
            const int64_t off = (b * H + h) * Dh;
            double *kc = kcache + (b * H + h) * W * Dh;
            double *vc = vcache + (b * H + h) * W * Dh;
            const double s = gate_sigmoid(gate_logit[h]);
            /* new entry */
            memcpy(rkl, k + off, (size_t)Dh * sizeof(double));
            rope_rotate(rkl, Dh, (double)p, rope_base, 0);
            memcpy(rk, kmem + off, (size_t)Dh * sizeof(double));
            rope_rotate(rk, Dh, (double)p, rope_base, 0);
            for (int c = 0; c < Dh; ++c) {
                double kn = rkl[c] + s * rk[c];
                double vn = v[off + c] + s * vmem[off + c];
                if (ring_bf16) { kn = oracle_round_bf16(kn); vn = oracle_round_bf16(vn); }
                kc[slot * Dh + c] = kn;
                vc[slot * Dh + c] = vn;
            }
            /* query */
            memcpy(qh, q + off, (size_t)Dh * sizeof(double));
            rope_rotate(qh, Dh, (double)p, rope_base, 0);
            double mx = -INFINITY;
            for (int64_t sl = 0; sl < W; ++sl) {
                const int64_t back = ((p - sl) % W + W) % W;
                if (p - back < 0) { sc[sl] = -INFINITY; continue; }
                sc[sl] = scale * dot(qh, kc + sl * Dh, Dh);
                if (sc[sl] > mx) mx = sc[sl];
            }
            double sum = 0.0;
            for (int64_t sl = 0; sl < W; ++sl) {
                sc[sl] = (sc[sl] == -INFINITY) ? 0.0 : exp(sc[sl] - mx);
                sum += sc[sl];
            }
            for (int c = 0; c < Dh; ++c) o[off + c] = 0.0;
            for (int64_t sl = 0; sl < W; ++sl) {
                if (sc[sl] == 0.0) continue;
                for (int c = 0; c < Dh; ++c) o[off + c] += sc[sl] / sum * vc[sl * Dh + c];
            }
            free(qh); free(rkl); free(rk); free(sc);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Row-sampled forward for large shapes: O and lse of the listed queries only.
 * rows[n] = (b, h, i) triples; o_rows [n][Dh]; lse_rows [n].
 * Computes the same quantities as oracle_swa_inject_fwd, one query at a time.
 * ------------------------------------------------------------------------- */
ORACLE_API void oracle_swa_inject_fwd_rows(int64_t B, int64_t T, int H, int Dh, int64_t W,
                                           int64_t pos0, double rope_base, double scale,
                                           const double *q, const double *k, const double *v,
                                           const double *kmem, const double *vmem,
                                           const double *gate_logit, int64_t nrows,
                                           const int64_t *rows, double *o_rows, double *lse_rows)
{
    (void)B;
    scale = default_scale(scale, Dh);
#pragma omp parallel for schedule(dynamic)
    for (int64_t n = 0; n < nrows; ++n) {
        const int64_t b = rows[3 * n], h = rows[3 * n + 1], i = rows[3 * n + 2];
        const double s = gate_sigmoid(gate_logit[h]);
        const int64_t lo = (i - W + 1) > 0 ? (i - W + 1) : 0;
        const int64_t cnt = i - lo + 1;
        double *kt = malloc((size_t)cnt * Dh * sizeof(double));
        double *vt = malloc((size_t)cnt * Dh * sizeof(double));
        double *qh = malloc((size_t)Dh * sizeof(double));
        double *rk = malloc((size_t)Dh * sizeof(double));
        double *p = malloc((size_t)cnt * sizeof(double));
        if (!kt || !vt || !qh || !rk || !p) abort();
        const int64_t qoff = ((b * T + i) * H + h) * Dh;
        memcpy(qh, q + qoff, (size_t)Dh * sizeof(double));
        rope_rotate(qh, Dh, (double)(pos0 + i), rope_base, 0);
        for (int64_t j = lo; j <= i; ++j) {
            const int64_t off = ((b * T + j) * H + h) * Dh;
            double *kj = kt + (j - lo) * Dh;
            memcpy(kj, k + off, (size_t)Dh * sizeof(double));
            rope_rotate(kj, Dh, (double)(pos0 + j), rope_base, 0);
            memcpy(rk, kmem + off, (size_t)Dh * sizeof(double));
            rope_rotate(rk, Dh, (double)(pos0 + j), rope_base, 0);
            for (int c = 0; c < Dh; ++c) {
                kj[c] += s * rk[c];
                vt[(j - lo) * Dh + c] = v[off + c] + s * vmem[off + c];
            }
        }
        double mx = -INFINITY;
        for (int64_t j = 0; j < cnt; ++j) {
            p[j] = scale * dot(qh, kt + j * Dh, Dh);
            if (p[j] > mx) mx = p[j];
        }
        double sum = 0.0;
        for (int64_t j = 0; j < cnt; ++j) { p[j] = exp(p[j] - mx); sum += p[j]; }
        for (int c = 0; c < Dh; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < cnt; ++j) acc += p[j] / sum * vt[j * Dh + c];
            o_rows[n * Dh + c] = acc;
        }
        if (lse_rows) lse_rows[n] = mx + log(sum);
        free(kt); free(vt); free(qh); free(rk); free(p);
    }
}

/* ===========================================================================
 * Gated variant ([R-step], the printed per-layer form):
 *     k^rec_t = RMSNorm(W_Km m'_{t-1}),       v^rec_t = W_Vm m'_{t-1},
 *     k~_t = g_kl (.) R_t k_t + g_kr (.) R_t k^rec_t,
 *     v~_t = g_vl (.) v_t     + g_vr (.) v^rec_t,
 *     g = 2 sigma(a)  (a = 0 gives the neutral value 1),
 * with one logit per channel of the H*Dh-wide key/value row for each of the
 * four gates. Readings where the page is silent: the RMSNorm runs over the
 * whole H*Dh projected row, has no learned scale of its own (the channel-wise
 * recurrent gate follows it) and adds eps inside the square root; the gates
 * multiply after the rotation, since the page rotates both kinds of key
 * before they are mixed ([R-bg]).
 * Gate vectors a_* are [H*Dh]; kproj is the pre-norm projection W_Km m'.
 * ========================================================================= */

/* Channel gate g = 2 sigma(a). */
static double gate_two_sigmoid(double a) { return 2.0 / (1.0 + exp(-a)); }

/* 1 / sqrt(mean(x^2) + eps) over n channels: the RMSNorm divisor's inverse. */
static double rms_inverse(const double *x, int n, double eps)
{
    return 1.0 / sqrt(dot(x, x, n) / (double)n + eps);
}

/* Mixed entries of one row (b, t): kmix/vmix [H*Dh] from k, v, kproj, vmem
 * rows of the same width; p is the absolute position. When rk_out/rn_out are
 * not NULL they receive R k and R RMSNorm(kproj) (both [H*Dh]). */
static void gated_row(int H, int Dh, double p, double base, double eps, const double *k,
                      const double *v, const double *kproj, const double *vmem,
                      const double *a_kl, const double *a_kr, const double *a_vl,
                      const double *a_vr, double *kmix, double *vmix, double *rk_out,
                      double *rn_out)
{
    const int HD = H * Dh;
    const double r = rms_inverse(kproj, HD, eps);
    double rk[512], rn[512];
    for (int h = 0; h < H; ++h) {
        const int o = h * Dh;
        memcpy(rk, k + o, (size_t)Dh * sizeof(double));
        rope_rotate(rk, Dh, p, base, 0);
        for (int c = 0; c < Dh; ++c) rn[c] = kproj[o + c] * r;
        rope_rotate(rn, Dh, p, base, 0);
        for (int c = 0; c < Dh; ++c) {
            kmix[o + c] = gate_two_sigmoid(a_kl[o + c]) * rk[c] +
                          gate_two_sigmoid(a_kr[o + c]) * rn[c];
            vmix[o + c] = gate_two_sigmoid(a_vl[o + c]) * v[o + c] +
                          gate_two_sigmoid(a_vr[o + c]) * vmem[o + c];
            if (rk_out) rk_out[o + c] = rk[c];
            if (rn_out) rn_out[o + c] = rn[c];
        }
    }
}

/* Gated mixed entries of every position; all activations [B,T,H,Dh]. */
ORACLE_API void oracle_gated_entries(int64_t B, int64_t T, int H, int Dh, int64_t pos0,
                                     double base, double eps, const double *k, const double *v,
                                     const double *kproj, const double *vmem,
                                     const double *a_kl, const double *a_kr,
                                     const double *a_vl, const double *a_vr, double *kmix,
                                     double *vmix)
{
    const int64_t HD = (int64_t)H * Dh;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t t = 0; t < T; ++t) {
            const int64_t off = (b * T + t) * HD;
            gated_row(H, Dh, (double)(pos0 + t), base, eps, k + off, v + off, kproj + off,
                      vmem + off, a_kl, a_kr, a_vl, a_vr, kmix + off, vmix + off, NULL, NULL);
        }
    }
}

/* q^ = R q and the given mixed entries of sequence (b, h), as a head view. */
static void head_view_entries(head_view *hv, int64_t b, int h, int64_t T, int H, int Dh,
                              int64_t pos0, double base, const double *q, const double *kmix,
                              const double *vmix)
{
    for (int64_t t = 0; t < T; ++t) {
        const int64_t off = ((b * T + t) * H + h) * Dh;
        double *qh = hv->qh + t * Dh;
        memcpy(qh, q + off, (size_t)Dh * sizeof(double));
        rope_rotate(qh, Dh, (double)(pos0 + t), base, 0);
        memcpy(hv->kt + t * Dh, kmix + off, (size_t)Dh * sizeof(double));
        memcpy(hv->vt + t * Dh, vmix + off, (size_t)Dh * sizeof(double));
    }
}

/* Sliding-window attention of the rotated queries over given mixed entries
 * (already rotated, already mixed): the attention half of the layer, whatever
 * the mixing form. o [B,T,H,Dh]; lse [B,H,T] (may be NULL). */
ORACLE_API void oracle_swa_attend_fwd(int64_t B, int64_t T, int H, int Dh, int64_t W,
                                      int64_t pos0, double rope_base, double scale,
                                      const double *q, const double *kmix, const double *vmix,
                                      double *o, double *lse)
{
    scale = default_scale(scale, Dh);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            head_view hv;
            double *p = malloc((size_t)(W < T ? W : T) * sizeof(double));
            if (!head_view_alloc(&hv, T, Dh) || !p) abort();
            head_view_entries(&hv, b, h, T, H, Dh, pos0, rope_base, q, kmix, vmix);
            for (int64_t i = 0; i < T; ++i) {
                double l;
                const int64_t lo = window_softmax(&hv, i, W, Dh, scale, p, &l);
                double *oi = o + ((b * T + i) * H + h) * Dh;
                for (int c = 0; c < Dh; ++c) oi[c] = 0.0;
                for (int64_t j = lo; j <= i; ++j)
                    for (int c = 0; c < Dh; ++c) oi[c] += p[j - lo] * hv.vt[j * Dh + c];
                if (lse) lse[((int64_t)b * H + h) * T + i] = l;
            }
            free(p);
            head_view_free(&hv);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Backward of the gated layer path (shift, projection, RMSNorm, gated mix,
 * attention), by the chain rule:
 *   outputs dq, dk, dv [B,T,H,Dh]; dm' [B,T,d]; dW_Km, dW_Vm [H*Dh,d];
 *           da_kl, da_kr, da_vl, da_vr [H*Dh] (summed over batch and time).
 * ------------------------------------------------------------------------- */
ORACLE_API void oracle_swa_inject_bwd_gated(int64_t B, int64_t T, int H, int Dh, int d,
                                            int64_t W, int64_t pos0, double rope_base,
                                            double scale, double eps, const double *q,
                                            const double *k, const double *v,
                                            const double *m_prime, const double *W_Km,
                                            const double *W_Vm, const double *a_kl,
                                            const double *a_kr, const double *a_vl,
                                            const double *a_vr, const double *dO, double *dq,
                                            double *dk, double *dv, double *dm_prime,
                                            double *dW_Km, double *dW_Vm, double *da_kl,
                                            double *da_kr, double *da_vl, double *da_vr)
{
    scale = default_scale(scale, Dh);
    const int HD = H * Dh;
    const size_t nact = (size_t)B * (size_t)T * (size_t)HD;
    double *kproj = malloc(nact * sizeof(double));
    double *vmem = malloc(nact * sizeof(double));
    double *kmix = malloc(nact * sizeof(double));
    double *vmix = malloc(nact * sizeof(double));
    double *dkmix = malloc(nact * sizeof(double));   /* d loss / d k~ (rotated frame) */
    double *dvmix = malloc(nact * sizeof(double));   /* d loss / d v~ */
    double *rk = malloc(nact * sizeof(double));      /* R k */
    double *rn = malloc(nact * sizeof(double));      /* R RMSNorm(kproj) */
    double *dkp = malloc(nact * sizeof(double));     /* d loss / d kproj */
    double *dvmem = malloc(nact * sizeof(double));   /* d loss / d vmem */
    if (!kproj || !vmem || !kmix || !vmix || !dkmix || !dvmix || !rk || !rn || !dkp || !dvmem)
        abort();

    oracle_mem_project(B, T, H, Dh, d, 1, m_prime, W_Km, W_Vm, kproj, vmem);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t t = 0; t < T; ++t) {
            const int64_t off = (b * T + t) * HD;
            gated_row(H, Dh, (double)(pos0 + t), rope_base, eps, k + off, v + off, kproj + off,
                      vmem + off, a_kl, a_kr, a_vl, a_vr, kmix + off, vmix + off, rk + off,
                      rn + off);
        }
    }

    /* attention: dq = R^T dq^, and the gradients of the mixed entries */
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            head_view hv;
            const int64_t wmax = W < T ? W : T;
            double *p = malloc((size_t)wmax * sizeof(double));
            double *dp = malloc((size_t)wmax * sizeof(double));
            double *dqh = calloc((size_t)T * Dh, sizeof(double));
            double *dkt = calloc((size_t)T * Dh, sizeof(double));
            double *dvt = calloc((size_t)T * Dh, sizeof(double));
            if (!head_view_alloc(&hv, T, Dh) || !p || !dp || !dqh || !dkt || !dvt) abort();
            head_view_entries(&hv, b, h, T, H, Dh, pos0, rope_base, q, kmix, vmix);
            for (int64_t i = 0; i < T; ++i) {
                const int64_t lo = window_softmax(&hv, i, W, Dh, scale, p, NULL);
                const double *dOi = dO + ((b * T + i) * H + h) * Dh;
                double Di = 0.0;
                for (int64_t j = lo; j <= i; ++j) {
                    dp[j - lo] = dot(dOi, hv.vt + j * Dh, Dh);
                    Di += p[j - lo] * dp[j - lo];
                }
                for (int64_t j = lo; j <= i; ++j) {
                    const double pij = p[j - lo];
                    const double dsij = pij * (dp[j - lo] - Di);
                    for (int c = 0; c < Dh; ++c) {
                        dqh[i * Dh + c] += scale * dsij * hv.kt[j * Dh + c];
                        dkt[j * Dh + c] += scale * dsij * hv.qh[i * Dh + c];
                        dvt[j * Dh + c] += pij * dOi[c];
                    }
                }
            }
            for (int64_t t = 0; t < T; ++t) {
                const int64_t off = ((b * T + t) * H + h) * Dh;
                rope_rotate(dqh + t * Dh, Dh, (double)(pos0 + t), rope_base, 1);
                memcpy(dq + off, dqh + t * Dh, (size_t)Dh * sizeof(double));
                memcpy(dkmix + off, dkt + t * Dh, (size_t)Dh * sizeof(double));
                memcpy(dvmix + off, dvt + t * Dh, (size_t)Dh * sizeof(double));
            }
            free(p); free(dp); free(dqh); free(dkt); free(dvt);
            head_view_free(&hv);
        }
    }

    /* gated mix and RMSNorm, row by row:
     *   dk   = R^T (g_kl (.) dk~),   dkn = R^T (g_kr (.) dk~)  (kn = kproj / rms)
     *   dkproj = (dkn - kn * mean(dkn (.) kn)) / rms           over the H*Dh row
     *   dv   = g_vl (.) dv~,         dvmem = g_vr (.) dv~ */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t t = 0; t < T; ++t) {
            const int64_t off = (b * T + t) * HD;
            const double pos = (double)(pos0 + t);
            const double r = rms_inverse(kproj + off, HD, eps);
            double tmp[512], dkn[4096];
            if (HD > 4096) abort();
            double mu = 0.0;
            for (int h = 0; h < H; ++h) {
                const int o = h * Dh;
                for (int c = 0; c < Dh; ++c) tmp[c] = gate_two_sigmoid(a_kl[o + c]) * dkmix[off + o + c];
                rope_rotate(tmp, Dh, pos, rope_base, 1);
                memcpy(dk + off + o, tmp, (size_t)Dh * sizeof(double));
                for (int c = 0; c < Dh; ++c) tmp[c] = gate_two_sigmoid(a_kr[o + c]) * dkmix[off + o + c];
                rope_rotate(tmp, Dh, pos, rope_base, 1);
                memcpy(dkn + o, tmp, (size_t)Dh * sizeof(double));
                for (int c = 0; c < Dh; ++c) {
                    dv[off + o + c] = gate_two_sigmoid(a_vl[o + c]) * dvmix[off + o + c];
                    dvmem[off + o + c] = gate_two_sigmoid(a_vr[o + c]) * dvmix[off + o + c];
                }
            }
            for (int c = 0; c < HD; ++c) mu += dkn[c] * kproj[off + c] * r;
            mu /= (double)HD;
            for (int c = 0; c < HD; ++c) dkp[off + c] = (dkn[c] - kproj[off + c] * r * mu) * r;
        }
    }

    /* gates: g = 2 sigma(a)  =>  dg/da = 2 sigma(a) (1 - sigma(a));
     *   d/dg_kl = sum dk~ (.) R k,   d/dg_kr = sum dk~ (.) R kn,
     *   d/dg_vl = sum dv~ (.) v,     d/dg_vr = sum dv~ (.) vmem  (over b, t) */
#pragma omp parallel for schedule(static)
    for (int c = 0; c < HD; ++c) {
        double gkl = 0.0, gkr = 0.0, gvl = 0.0, gvr = 0.0;
        for (int64_t n = 0; n < B * T; ++n) {
            const int64_t i = n * HD + c;
            gkl += dkmix[i] * rk[i];
            gkr += dkmix[i] * rn[i];
            gvl += dvmix[i] * v[i];
            gvr += dvmix[i] * vmem[i];
        }
        const double skl = gate_sigmoid(a_kl[c]), skr = gate_sigmoid(a_kr[c]);
        const double svl = gate_sigmoid(a_vl[c]), svr = gate_sigmoid(a_vr[c]);
        da_kl[c] = 2.0 * skl * (1.0 - skl) * gkl;
        da_kr[c] = 2.0 * skr * (1.0 - skr) * gkr;
        da_vl[c] = 2.0 * svl * (1.0 - svl) * gvl;
        da_vr[c] = 2.0 * svr * (1.0 - svr) * gvr;
    }

    /* shift and projection, as in the ungated backward: row t of the
     * projection input is m'[t-1]; dm'[T-1] = 0 */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t t = 0; t < T; ++t) {
            double *out = dm_prime + (b * T + t) * d;
            if (t == T - 1) {
                for (int e = 0; e < d; ++e) out[e] = 0.0;
                continue;
            }
            const double *gk = dkp + (b * T + t + 1) * HD;
            const double *gv = dvmem + (b * T + t + 1) * HD;
            for (int e = 0; e < d; ++e) {
                double acc = 0.0;
                for (int r = 0; r < HD; ++r)
                    acc += gk[r] * W_Km[(int64_t)r * d + e] + gv[r] * W_Vm[(int64_t)r * d + e];
                out[e] = acc;
            }
        }
    }
#pragma omp parallel for schedule(static)
    for (int r = 0; r < HD; ++r) {
        for (int e = 0; e < d; ++e) {
            double ak = 0.0, av = 0.0;
            for (int64_t b = 0; b < B; ++b) {
                for (int64_t t = 1; t < T; ++t) {
                    const double x = m_prime[(b * T + t - 1) * d + e];
                    ak += dkp[(b * T + t) * HD + r] * x;
                    av += dvmem[(b * T + t) * HD + r] * x;
                }
            }
            dW_Km[(int64_t)r * d + e] = ak;
            dW_Vm[(int64_t)r * d + e] = av;
        }
    }
    free(kproj); free(vmem); free(kmix); free(vmix); free(dkmix); free(dvmix);
    free(rk); free(rn); free(dkp); free(dvmem);
}

/* ---------------------------------------------------------------------------
 * One recurrent decode step of the gated variant on a W-slot ring: the new
 * entry of stream b is the gated mix of its row (kproj = W_Km m_{t-1} before
 * the norm, vmem = W_Vm m_{t-1}) at position pos[b], written to slot
 * pos mod W (bf16-rounded when ring_bf16 != 0); then the rotated query
 * attends over the valid slots, as in the ungated step.
 * q,k,v,kproj,vmem,o [Bs,H,Dh]; caches [Bs,H,W,Dh] (in/out).
 * ------------------------------------------------------------------------- */
ORACLE_API void oracle_decode_step_gated(int64_t Bs, int H, int Dh, int64_t W, double rope_base,
                                         double scale, double eps, int ring_bf16,
                                         const double *q, const double *k, const double *v,
                                         const double *kproj, const double *vmem,
                                         const double *a_kl, const double *a_kr,
                                         const double *a_vl, const double *a_vr,
                                         double *kcache, double *vcache, const int64_t *pos,
                                         double *o)
{
    scale = default_scale(scale, Dh);
    const int HD = H * Dh;
    double *kn = malloc((size_t)Bs * HD * sizeof(double));
    double *vn = malloc((size_t)Bs * HD * sizeof(double));
    if (!kn || !vn) abort();
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < Bs; ++b) {
        const int64_t off = b * HD;
        gated_row(H, Dh, (double)pos[b], rope_base, eps, k + off, v + off, kproj + off,
                  vmem + off, a_kl, a_kr, a_vl, a_vr, kn + off, vn + off, NULL, NULL);
    }
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < Bs; ++b) {
        for (int h = 0; h < H; ++h) {
            double *qh = malloc((size_t)Dh * sizeof(double));
            double *sc = malloc((size_t)W * sizeof(double));
            if (!qh || !sc) abort();
            const int64_t p = pos[b];
            const int64_t slot = p % W;
            const int64_t off = (b * H + h) * Dh;
            double *kc = kcache + (b * H + h) * W * Dh;
            double *vc = vcache + (b * H + h) * W * Dh;
            for (int c = 0; c < Dh; ++c) {
                double ke = kn[off + c], ve = vn[off + c];
                if (ring_bf16) { ke = oracle_round_bf16(ke); ve = oracle_round_bf16(ve); }
                kc[slot * Dh + c] = ke;
                vc[slot * Dh + c] = ve;
            }
            memcpy(qh, q + off, (size_t)Dh * sizeof(double));
            rope_rotate(qh, Dh, (double)p, rope_base, 0);
            double mx = -INFINITY;
            for (int64_t sl = 0; sl < W; ++sl) {
                const int64_t back = ((p - sl) % W + W) % W;
                if (p - back < 0) { sc[sl] = -INFINITY; continue; }
                sc[sl] = scale * dot(qh, kc + sl * Dh, Dh);
                if (sc[sl] > mx) mx = sc[sl];
            }
            double sum = 0.0;
            for (int64_t sl = 0; sl < W; ++sl) {
                sc[sl] = (sc[sl] == -INFINITY) ? 0.0 : exp(sc[sl] - mx);
                sum += sc[sl];
            }
            for (int c = 0; c < Dh; ++c) o[off + c] = 0.0;
            for (int64_t sl = 0; sl < W; ++sl) {
                if (sc[sl] == 0.0) continue;
                for (int c = 0; c < Dh; ++c) o[off + c] += sc[sl] / sum * vc[sl * Dh + c];
            }
            free(qh); free(sc);
        }
    }
    free(kn); free(vn);
}

/* ===========================================================================
 * Loss head ([R-step]: the output state m_t feeds the LM head
 * p(x_{t+1} | x_{<=t}) = softmax(cap * tanh(U m_t / cap)) with cap = 15, and
 * the loss is the mean over positions of CE + lambda ||m_t - m'_t||^2 / sqrt(d);
 * the targets m' are states after the final RMSNorm, so m_t is taken as the
 * final RMSNorm of the decoder's last hidden state h_t).
 *   m_n   = h_n / sqrt(mean(h_n^2) + eps)            (no learned scale)
 *   c_nv  = cap tanh((U m_n)_v / cap)
 *   CE_n  = log sum_v exp(c_nv) - c_n,target_n        (0 when the target is
 *           outside [0, V): the position is ignored; N still divides)
 *   loss  = sum_n CE_n / N + lambda / (N sqrt(d)) sum_n ||m_n - m'_n||^2
 * Gradients by the chain rule: dc = (softmax(c) - onehot) / N,
 *   dz = dc (1 - tanh^2), dm = U^T dz + 2 lambda (m - m') / (N sqrt d),
 *   dU = sum_n dz_n m_n^T, dh = r (dm - m mean(dm (.) m)), r = 1 / rms(h).
 * h, m, m' [N,d]; U [V,d]; targets [N]; dh [N,d]; dU [V,d] (may be NULL);
 * m_prime may be NULL (no consistency term). Returns the loss.
 * ========================================================================= */
ORACLE_API double oracle_lm_head(int64_t N, int d, int64_t V, double cap, double eps,
                                 double lambda, const double *h, const double *U,
                                 const int64_t *targets, const double *m_prime, double *m_out,
                                 double *dh, double *dU)
{
    double *m = malloc((size_t)N * d * sizeof(double));
    double *rr = malloc((size_t)N * sizeof(double));
    double *ce = malloc((size_t)N * sizeof(double));
    double *dz = dU ? malloc((size_t)N * V * sizeof(double)) : NULL;
    if (!m || !rr || !ce || (dU && !dz)) abort();
    const double cons = m_prime ? lambda / ((double)N * sqrt((double)d)) : 0.0;
#pragma omp parallel for schedule(dynamic)
    for (int64_t n = 0; n < N; ++n) {
        const double *hn = h + n * d;
        double *mn = m + n * d;
        const double r = 1.0 / sqrt(dot(hn, hn, d) / (double)d + eps);
        rr[n] = r;
        for (int e = 0; e < d; ++e) mn[e] = hn[e] * r;
        double *c = malloc((size_t)V * sizeof(double));
        double *dm = malloc((size_t)d * sizeof(double));
        if (!c || !dm) abort();
        double mx = -INFINITY;
        for (int64_t v = 0; v < V; ++v) {
            c[v] = cap * tanh(dot(U + v * d, mn, d) / cap);
            if (c[v] > mx) mx = c[v];
        }
        double sum = 0.0;
        for (int64_t v = 0; v < V; ++v) sum += exp(c[v] - mx);
        const double lse = mx + log(sum);
        const int64_t tgt = targets[n];
        const int valid = tgt >= 0 && tgt < V;
        ce[n] = valid ? lse - c[tgt] : 0.0;
        /* dm = U^T dz (+ consistency) */
        for (int e = 0; e < d; ++e)
            dm[e] = m_prime ? 2.0 * cons * (mn[e] - m_prime[n * d + e]) : 0.0;
        for (int64_t v = 0; v < V; ++v) {
            const double t = c[v] / cap;
            double g = valid ? (exp(c[v] - lse) - (v == tgt ? 1.0 : 0.0)) / (double)N : 0.0;
            g *= (1.0 - t * t);
            if (dz) dz[n * V + v] = g;
            for (int e = 0; e < d; ++e) dm[e] += g * U[v * d + e];
        }
        if (dh) {
            const double mu = dot(dm, mn, d) / (double)d;
            for (int e = 0; e < d; ++e) dh[n * d + e] = r * (dm[e] - mn[e] * mu);
        }
        free(c); free(dm);
    }
    if (dU) {
#pragma omp parallel for schedule(static)
        for (int64_t v = 0; v < V; ++v)
            for (int e = 0; e < d; ++e) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) acc += dz[n * V + v] * m[n * d + e];
                dU[v * d + e] = acc;
            }
    }
    double loss = 0.0;
    for (int64_t n = 0; n < N; ++n) loss += ce[n];
    loss /= (double)N;
    if (m_prime)
        for (int64_t i = 0; i < N * (int64_t)d; ++i) {
            const double diff = m[i] - m_prime[i];
            loss += cons * diff * diff;
        }
    if (m_out) memcpy(m_out, m, (size_t)N * d * sizeof(double));
    free(m); free(rr); free(ce); free(dz);
    return loss;
}

/* Per-row quantities of the loss head for listed rows only (for large
 * shapes): the log-sum-exp of row n's capped logits, its CE term and the
 * head's part of dm_n (U^T dz_n, no consistency term), for rows[i]. */
ORACLE_API void oracle_lm_head_rows(int64_t nrows, const int64_t *rows, int d, int64_t V,
                                    double cap, double eps, int64_t N, const double *h,
                                    const double *U, const int64_t *targets, double *lse_out,
                                    double *ce_out, double *dm_out)
{
#pragma omp parallel for schedule(dynamic)
    for (int64_t i = 0; i < nrows; ++i) {
        const int64_t n = rows[i];
        const double *hn = h + n * d;
        double *mn = malloc((size_t)d * sizeof(double));
        double *c = malloc((size_t)V * sizeof(double));
        if (!mn || !c) abort();
        const double r = 1.0 / sqrt(dot(hn, hn, d) / (double)d + eps);
        for (int e = 0; e < d; ++e) mn[e] = hn[e] * r;
        double mx = -INFINITY;
        for (int64_t v = 0; v < V; ++v) {
            c[v] = cap * tanh(dot(U + v * d, mn, d) / cap);
            if (c[v] > mx) mx = c[v];
        }
        double sum = 0.0;
        for (int64_t v = 0; v < V; ++v) sum += exp(c[v] - mx);
        const double lse = mx + log(sum);
        const int64_t tgt = targets[n];
        const int valid = tgt >= 0 && tgt < V;
        lse_out[i] = lse;
        ce_out[i] = valid ? lse - c[tgt] : 0.0;
        for (int e = 0; e < d; ++e) dm_out[i * d + e] = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            const double t = c[v] / cap;
            const double g = valid ? (exp(c[v] - lse) - (v == tgt ? 1.0 : 0.0)) / (double)N
                                       * (1.0 - t * t) : 0.0;
            for (int e = 0; e < d; ++e) dm_out[i * d + e] += g * U[v * d + e];
        }
        free(mn); free(c);
    }
}
