/*
 * oracle.c -- plain, slow fp64 CPU oracle of the DeepSeek-V3-style MoE layer
 * forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (the HIP library) never calls it, and the two share no code: this file has
 * its own decoders, selection, permutation, FFN and quantiser.
 *
 * Sources (cited by page title and section):
 *   [Co-design]  "从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计"
 *                (wsisp.com/helps/120648.html).  Section 2.2 prints the
 *                MoEGate module; section 2.3 prints the dispatch skeleton.
 *   [Insights]   "深入理解 DeepSeek-V3：大规模缩放挑战与对 AI 架构硬件的反思（中文精读）"
 *                (digest of arXiv 2505.09343).  Section 3.1: 8 routed + 1
 *                shared expert per token; section 3.2: FP8 with 1x128
 *                activation tiles and 128x128 weight blocks.
 *   [mqxn]       mqxn.cn/news/19449, section 3.1: the FFN is SwiGLU.
 *
 * Readings where the pages are silent or ambiguous (each is repeated at the
 * step it affects; R8-R10 concern only the GPU path and are not listed):
 *   R1  ties in every top-k go to the lower index; the top_k slots are in
 *       descending order of the masked choice score (the printed code uses
 *       topk(..., sorted=False), which fixes neither).
 *   R2  experts outside the kept groups get choice score 0.0, as printed
 *       (not -inf), so they can still win against negative scores.
 *   R3  normalisation only when top_k > 1; the routed scaling factor always.
 *   R4  the token sort by expert id is stable (ascending flat index inside
 *       an expert).
 *   R5  SwiGLU expert: W2 (silu(W_gate x) * (W_up x)), no biases; gate rows
 *       first, up rows second in the stacked W13.
 *   R6  layer output = shared(x) + sum_k w_k expert_k(x); the shared expert is
 *       unweighted; no residual or norm inside the layer.
 *   R7  FP8 scale of a tile with max |v| = a: scale = a / 448, codes are the
 *       e4m3 values nearest v * (448 / a) (ties to even, saturating);
 *       an all-zero tile has scale 1 and zero codes.
 *   R14 FP8 with power-of-two scales ([Insights] 3.2 asks for matrix units
 *       that take the block scales themselves; such units take scales that
 *       are powers of two): the scale of a tile is the smallest power of two
 *       2^e >= a / 448 (e clamped to [-126, 127]), codes are the e4m3 values
 *       nearest v * 2^-e (an exact product; ties to even); an all-zero tile
 *       has scale 1 and zero codes.
 *   R15 the FP8 backward ([Insights] 3.2 fixes the granularity of FP8
 *       training -- activations in 1x128 tiles, weights in 128x128 blocks,
 *       fp32 accumulation -- and says no more about the backward): every
 *       operand of a backward GEMM that is an activation or a gradient is
 *       quantised in tiles of 128 along that GEMM's contraction dimension
 *       (for the weight gradients, which contract over an expert's rows:
 *       128 consecutive rows of one column); the weights keep their 128x128
 *       blocks; the forward quantities are recomputed as the FP8 forward
 *       computes them.
 *   R11 the selection bias follows the experts' observed load ([Co-design]
 *       2.2 keeps it as a buffer updated from load statistics, not from a
 *       gradient, and prints no rule): each expert's bias moves one fixed
 *       step gamma toward balance -- up when the expert received fewer rows
 *       than the mean over experts, down when more, unchanged at exactly the
 *       mean.  The bias is an fp32 buffer; the step is rounded once to fp32.
 *
 * Every floating-point step here is in double unless it is marked as the
 * fp32 selection contract.  Compile without floating-point contraction.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3 = 2 };

typedef struct {
    int32_t H;   /* hidden size                         */
    int32_t E;   /* n_routed_experts                    */
    int32_t G;   /* n_group                             */
    int32_t TG;  /* topk_group                          */
    int32_t K;   /* num_experts_per_tok (top_k)         */
    int32_t I;   /* routed expert intermediate size     */
    int32_t Is;  /* shared expert intermediate size     */
    double rho;  /* routed_scaling_factor               */
} oracle_cfg;

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- number formats ---------------------------------------------------- */

/* bf16 is the upper 16 bits of an IEEE binary32; widening is exact. */
static double dec_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP 8-bit e4m3fn: sign bit, 4-bit exponent with bias 7, 3-bit mantissa.
 * Exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no inf. */
double oracle_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest e4m3 code to v: bisection over the 127 non-negative finite codes
 * (their values increase with the code), ties to the even code (even
 * mantissa), magnitudes beyond 448 saturate to 448 (R7). */
uint8_t oracle_e4m3_encode(float v)
{
    double a = fabs((double)v);
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (a >= 448.0)
        return sign | 0x7E;
    int lo = 0, hi = 0x7E;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (oracle_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - oracle_e4m3_decode((uint8_t)lo);
    double dhi = oracle_e4m3_decode((uint8_t)hi) - a;
    int code = (dlo < dhi) ? lo : (dhi < dlo) ? hi : ((lo % 2 == 0) ? lo : hi);
    return sign | (uint8_t)code;
}

/* Element (r, c) of a row-major [rows, cols] matrix stored as dtype dt.
 * e4m3 matrices carry one fp32 scale per 128x128 block, [rows/128, cols/128]
 * row-major ([Insights] 3.2: weights in 128x128 blocks). */
static double mat_at(const void *base, const float *scale, int dt, int64_t cols,
                     int64_t r, int64_t c)
{
    int64_t i = r * cols + c;
    switch (dt) {
    case OR_F32:
        return (double)((const float *)base)[i];
    case OR_BF16:
        return dec_bf16(((const uint16_t *)base)[i]);
    default: {
        double q = oracle_e4m3_decode(((const uint8_t *)base)[i]);
        return q * (double)scale[(r / 128) * (cols / 128) + c / 128];
    }
    }
}

/* ---- FP8 activation quantiser ([Insights] 3.2: 1x128 activation tiles) - */

/* Each row of v [rows, cols] (cols % 128 == 0) in tiles of 128: a = max |v|;
 * scale = a / 448 rounded to float; inv = 448 / a rounded to float; code =
 * nearest e4m3 of the float product v * inv (R7).  s is [rows, cols/128]. */
void oracle_quant_rows(int64_t rows, int32_t cols, const float *v, uint8_t *q, float *s)
{
    int32_t nt = cols / 128;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int32_t t = 0; t < nt; ++t) {
            const float *p = v + r * cols + (int64_t)t * 128;
            double a = 0.0;
            for (int j = 0; j < 128; ++j)
                if (fabs((double)p[j]) > a)
                    a = fabs((double)p[j]);
            float scale = 1.0f, inv = 0.0f;
            if (a > 0.0) {
                scale = (float)(a / 448.0);
                inv = (float)(448.0 / a);
            }
            s[r * nt + t] = scale;
            for (int j = 0; j < 128; ++j) {
                float prod = p[j] * inv; /* one fp32 multiply */
                q[r * cols + (int64_t)t * 128 + j] = oracle_e4m3_encode(prod);
            }
        }
    }
}

/* Power-of-two scale of a tile with max |v| = a > 0 (R14): the smallest
 * 2^e with 2^e >= a / 448.  a / 448 in double is a power of two exactly when
 * a is 7 * 2^k (448 = 7 * 2^6), and is then computed exactly; frexp gives
 * a / 448 = f * 2^ex with f in [0.5, 1), a power of two iff f == 0.5. */
static int pow2_scale_exponent(double a)
{
    int ex;
    double f = frexp(a / 448.0, &ex);
    int e = (f == 0.5) ? ex - 1 : ex;
    if (e < -126)
        e = -126;
    if (e > 127)
        e = 127;
    return e;
}

/* The same 1x128 quantiser with power-of-two scales (R14). */
void oracle_quant_rows_pow2(int64_t rows, int32_t cols, const float *v, uint8_t *q, float *s)
{
    int32_t nt = cols / 128;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int32_t t = 0; t < nt; ++t) {
            const float *p = v + r * cols + (int64_t)t * 128;
            double a = 0.0;
            for (int j = 0; j < 128; ++j)
                if (fabs((double)p[j]) > a)
                    a = fabs((double)p[j]);
            float scale = 1.0f, inv = 0.0f;
            if (a > 0.0) {
                int e = pow2_scale_exponent(a);
                scale = (float)ldexp(1.0, e);
                inv = (float)ldexp(1.0, -e);
            }
            s[r * nt + t] = scale;
            for (int j = 0; j < 128; ++j) {
                float prod = p[j] * inv; /* exact: inv is a power of two */
                q[r * cols + (int64_t)t * 128 + j] = oracle_e4m3_encode(prod);
            }
        }
    }
}

/* Activation quantisation modes of the layer functions. */
enum { OR_QUANT_NONE = 0, OR_QUANT_AMAX = 1, OR_QUANT_POW2 = 2 };

/* Quantise then dequantise one row in place (double in, double out) with the
 * scale rule of `mode` (R7 or R14). */
static void quant_dequant_row(double *v, int32_t n, int32_t mode)
{
    float tmp[128];
    uint8_t q[128];
    float s;
    for (int32_t t = 0; t < n / 128; ++t) {
        for (int j = 0; j < 128; ++j)
            tmp[j] = (float)v[t * 128 + j];
        if (mode == OR_QUANT_POW2)
            oracle_quant_rows_pow2(1, 128, tmp, q, &s);
        else
            oracle_quant_rows(1, 128, tmp, q, &s);
        for (int j = 0; j < 128; ++j)
            v[t * 128 + j] = oracle_e4m3_decode(q[j]) * (double)s;
    }
}

/* ---- step 1: gate logits ([Co-design] 2.2, MoEGate.forward: a linear map
 *      of the fp32-cast hidden states by the gate weight) ------------------ */

void oracle_logits(int64_t T, int32_t H, int32_t E, const void *x, int32_t x_dtype,
                   const float *gate_w, double *logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int32_t h = 0; h < H; ++h)
                acc += mat_at(x, NULL, x_dtype, H, t, h) * (double)gate_w[(int64_t)e * H + h];
            logits[t * E + e] = acc;
        }
    }
}

/* ---- steps 2-8: scores, choice scores, group limit, top-k, weights ------ */

/* Index of the largest v[i] over i in [0, n) with taken[i] == 0; ties go to
 * the lower index (R1). */
static int argmax_free_d(const double *v, const unsigned char *taken, int n)
{
    int best = -1;
    for (int i = 0; i < n; ++i)
        if (!taken[i] && (best < 0 || v[i] > v[best]))
            best = i;
    return best;
}

static int argmax_free_f(const float *v, const unsigned char *taken, int n)
{
    int best = -1;
    for (int i = 0; i < n; ++i)
        if (!taken[i] && (best < 0 || v[i] > v[best]))
            best = i;
    return best;
}

static int check_cfg(const oracle_cfg *c)
{
    if (c->E <= 0 || c->G <= 0 || c->E % c->G != 0 || c->E / c->G < 2)
        return 1;
    if (c->TG < 1 || c->TG > c->G || c->K < 1 || c->K > c->E)
        return 1;
    return 0;
}

/* Router in double precision.  For every token:
 *   s = sigmoid(l)                                  [Co-design] 2.2 (scores)
 *   c = s + bias  (bias only chooses)               [Co-design] 2.2 (scores_for_choice)
 *   g_j = sum of the two largest c in group j;      [Co-design] 2.2 (group_scores:
 *         group j = experts [j E/G, (j+1) E/G)        view as (n_group, E/G), top 2, sum)
 *   keep the TG groups with the largest g           [Co-design] 2.2 (group_idx)
 *   c' = c inside kept groups, else 0.0 (R2)        [Co-design] 2.2 (tmp_scores)
 *   idx = the K largest c' (R1)                     [Co-design] 2.2 (topk_idx)
 *   w = s[idx]; if K > 1: w /= (sum w + 1e-20); w *= rho (R3)
 *                                                   [Co-design] 2.2 (topk_weight)
 * margin[t] = the smaller of the gap between the TG-th and (TG+1)-th group
 * score and the gap between the K-th and (K+1)-th masked choice score
 * (+inf where there is no such boundary): how far the token is from a
 * different selection. */
int oracle_route_f64(const oracle_cfg *c, int64_t T, const double *logits, const float *bias,
                     int32_t *idx, double *w, double *margin)
{
    if (check_cfg(c))
        return 1;
    const int E = c->E, G = c->G, Eg = c->E / c->G, TG = c->TG, K = c->K;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t t = 0; t < T; ++t) {
        double *s = malloc(sizeof(double) * E), *ch = malloc(sizeof(double) * E);
        double *cm = malloc(sizeof(double) * E), *g = malloc(sizeof(double) * G);
        unsigned char *taken = malloc(E > G ? E : G), *keep = malloc(G);
        if (!s || !ch || !cm || !g || !taken || !keep) {
            bad = 1;
        } else {
            for (int e = 0; e < E; ++e) {
                s[e] = 1.0 / (1.0 + exp(-logits[t * E + e]));
                ch[e] = s[e] + (double)bias[e];
            }
            for (int j = 0; j < G; ++j) {
                memset(taken, 0, Eg);
                int a = argmax_free_d(ch + j * Eg, taken, Eg); /* Eg >= 2 */
                taken[a < 0 ? 0 : a] = 1;
                int b = argmax_free_d(ch + j * Eg, taken, Eg);
                g[j] = ch[j * Eg + a] + ch[j * Eg + b];
            }
            memset(taken, 0, G);
            memset(keep, 0, G);
            double last_g = 0.0;
            for (int r = 0; r < TG; ++r) {
                int j = argmax_free_d(g, taken, G);
                taken[j] = 1;
                keep[j] = 1;
                last_g = g[j];
            }
            double m = INFINITY;
            if (TG < G) {
                int j = argmax_free_d(g, taken, G);
                m = last_g - g[j];
            }
            for (int e = 0; e < E; ++e)
                cm[e] = keep[e / Eg] ? ch[e] : 0.0;
            memset(taken, 0, E);
            double last_c = 0.0, sum = 0.0;
            for (int k = 0; k < K; ++k) {
                int e = argmax_free_d(cm, taken, E);
                taken[e] = 1;
                idx[t * K + k] = e;
                w[t * K + k] = s[e];
                sum += s[e];
                last_c = cm[e];
            }
            if (K < E) {
                int e = argmax_free_d(cm, taken, E);
                if (last_c - cm[e] < m)
                    m = last_c - cm[e];
            }
            for (int k = 0; k < K; ++k) {
                if (K > 1)
                    w[t * K + k] = w[t * K + k] / (sum + 1e-20);
                w[t * K + k] = w[t * K + k] * c->rho;
            }
            if (margin)
                margin[t] = m;
        }
        free(s); free(ch); free(cm); free(g); free(taken); free(keep);
    }
    return bad ? 2 : 0;
}

/* Router under the fp32 selection contract, from fp32 logits L:
 *   s32 = fp32 rounding of the double sigmoid 1 / (1 + exp(-L))
 *   c32 = s32 + bias (one fp32 add)
 *   g32 = c32_(1) + c32_(2) (one fp32 add of the group's two largest)
 *   selections by exact fp32 comparison, ties to the lower index (R1),
 *   masked experts +0.0f (R2).
 * The steps and their order are those of oracle_route_f64; only the
 * precision of the decision differs, so that a caller holding fp32 logits
 * can reproduce the decision bit for bit.  Weights are returned in double,
 * from the double sigmoid of L (R3). */
int oracle_route_f32(const oracle_cfg *c, int64_t T, const float *logits, const float *bias,
                     int32_t *idx, double *w)
{
    if (check_cfg(c))
        return 1;
    const int E = c->E, G = c->G, Eg = c->E / c->G, TG = c->TG, K = c->K;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t t = 0; t < T; ++t) {
        double *s = malloc(sizeof(double) * E);
        float *ch = malloc(sizeof(float) * E), *cm = malloc(sizeof(float) * E);
        float *g = malloc(sizeof(float) * G);
        unsigned char *taken = malloc(E > G ? E : G), *keep = malloc(G);
        if (!s || !ch || !cm || !g || !taken || !keep) {
            bad = 1;
        } else {
            for (int e = 0; e < E; ++e) {
                s[e] = 1.0 / (1.0 + exp(-(double)logits[t * E + e]));
                float s32 = (float)s[e];
                ch[e] = s32 + bias[e];
            }
            for (int j = 0; j < G; ++j) {
                memset(taken, 0, Eg);
                int a = argmax_free_f(ch + j * Eg, taken, Eg); /* Eg >= 2 */
                taken[a < 0 ? 0 : a] = 1;
                int b = argmax_free_f(ch + j * Eg, taken, Eg);
                g[j] = ch[j * Eg + a] + ch[j * Eg + b];
            }
            memset(taken, 0, G);
            memset(keep, 0, G);
            for (int r = 0; r < TG; ++r) {
                int j = argmax_free_f(g, taken, G);
                taken[j] = 1;
                keep[j] = 1;
            }
            for (int e = 0; e < E; ++e)
                cm[e] = keep[e / Eg] ? ch[e] : 0.0f;
            memset(taken, 0, E);
            double sum = 0.0;
            for (int k = 0; k < K; ++k) {
                int e = argmax_free_f(cm, taken, E);
                taken[e] = 1;
                idx[t * K + k] = e;
                w[t * K + k] = s[e];
                sum += s[e];
            }
            for (int k = 0; k < K; ++k) {
                if (K > 1)
                    w[t * K + k] = w[t * K + k] / (sum + 1e-20);
                w[t * K + k] = w[t * K + k] * c->rho;
            }
        }
        free(s); free(ch); free(cm); free(g); free(taken); free(keep);
    }
    return bad ? 2 : 0;
}

/* ---- steps 9-10: per-expert counts and the token order ([Co-design] 2.3:
 *      one-hot counts summed per expert; argsort of the flattened expert
 *      ids; rows gathered as x[order // top_k]) ---------------------------- */

/* counts[e] = #{f : idx[f] == e}; offsets = exclusive prefix sum with
 * offsets[E] = T*K; perm lists the flat indices f = t*K + k grouped by
 * expert, ascending f inside an expert (a stable counting sort, R4);
 * pos[perm[j]] = j.  Returns 1 if an index is out of range. */
int oracle_permute(int64_t T, int32_t K, int32_t E, const int32_t *idx, int32_t *counts,
                   int32_t *offsets, int32_t *perm, int32_t *pos)
{
    int64_t N = T * K;
    for (int32_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t f = 0; f < N; ++f) {
        if (idx[f] < 0 || idx[f] >= E)
            return 1;
        counts[idx[f]] += 1;
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *next = malloc(sizeof(int32_t) * (E > 0 ? E : 1));
    if (!next)
        return 2;
    memcpy(next, offsets, sizeof(int32_t) * E);
    for (int64_t f = 0; f < N; ++f) {
        int32_t j = next[idx[f]]++;
        perm[j] = (int32_t)f;
        pos[f] = j;
    }
    free(next);
    return 0;
}

/* ---- steps 11-13: expert FFNs and the combine --------------------------- */

/* One SwiGLU FFN on one row (R5): a = W13 x (2n rows: gate then up),
 * h = silu(a[:n]) * a[n:], silu(z) = z / (1 + exp(-z)), y = W2 h.
 * W13 is [2n, H], W2 is [H, n].  quant_h: quantise h per 1x128 first, with
 * the scale rule of that mode (OR_QUANT_AMAX: R7, OR_QUANT_POW2: R14). */
static void ffn_row(int32_t H, int32_t n, const double *xrow, const void *w13,
                    const float *s13, const void *w2, const float *s2, int dt,
                    int quant_h, double *h, double *y)
{
    for (int32_t i = 0; i < n; ++i) {
        double gsum = 0.0, usum = 0.0;
        for (int32_t k = 0; k < H; ++k) {
            gsum += mat_at(w13, s13, dt, H, i, k) * xrow[k];
            usum += mat_at(w13, s13, dt, H, n + i, k) * xrow[k];
        }
        h[i] = gsum / (1.0 + exp(-gsum)) * usum;
    }
    if (quant_h)
        quant_dequant_row(h, n, quant_h);
    for (int32_t m = 0; m < H; ++m) {
        double acc = 0.0;
        for (int32_t i = 0; i < n; ++i)
            acc += mat_at(w2, s2, dt, n, m, i) * h[i];
        y[m] = acc;
    }
}

static const void *expert_base(const void *w, int dt, int64_t e, int64_t elems)
{
    size_t sz = (dt == OR_F32) ? 4 : (dt == OR_BF16) ? 2 : 1;
    return (const char *)w + (size_t)(e * elems) * sz;
}

/* Layer output for the listed tokens (R6):
 *   out[t] = shared(x_t) + sum_k w[t,k] * expert_{idx[t,k]}(x_t)
 * ([Co-design] 2.2: the shared expert is always active; [Insights] 3.1:
 * 8 routed + 1 shared per token; [Co-design] 2.3: expert results are
 * collected back to their tokens).  Expert e's output on token t is the
 * row that the sorted-token layout holds at pos[t*K+k], so it is evaluated
 * directly on x_t here.  w13 is [E, 2I, H], w2 [E, H, I], ws13 [2Is, H],
 * ws2 [H, Is]; e4m3 weights use 128x128 block scales (the dequantised
 * weights are the layer's weights).  quant_act: also quantise x and h per
 * 1x128 tile as the FP8 data path does (OR_QUANT_AMAX: scales a / 448, R7;
 * OR_QUANT_POW2: power-of-two scales, R14).
 * out is [n_tok, H]. */
int oracle_layer(const oracle_cfg *c, int64_t n_tok, const int64_t *tokens, const void *x,
                 int32_t x_dtype, const int32_t *idx, const double *w, const void *w13,
                 const float *w13_s, const void *w2, const float *w2_s, const void *ws13,
                 const float *ws13_s, const void *ws2, const float *ws2_s, int32_t w_dtype,
                 int32_t quant_act, double *out)
{
    const int32_t H = c->H, I = c->I, Is = c->Is, K = c->K, E = c->E;
    int bad = 0;
    int32_t nmax = I > Is ? I : Is;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t n = 0; n < n_tok; ++n) {
        int64_t t = tokens[n];
        double *xr = malloc(sizeof(double) * H), *y = malloc(sizeof(double) * H);
        double *h = malloc(sizeof(double) * (nmax > 0 ? nmax : 1));
        double *o = out + n * H;
        if (!xr || !y || !h) {
            bad = 1;
        } else {
            for (int32_t k = 0; k < H; ++k)
                xr[k] = mat_at(x, NULL, x_dtype, H, t, k);
            if (quant_act)
                quant_dequant_row(xr, H, quant_act);
            for (int32_t k = 0; k < H; ++k)
                o[k] = 0.0;
            if (Is > 0) {
                ffn_row(H, Is, xr, ws13, ws13_s, ws2, ws2_s, w_dtype, quant_act, h, y);
                for (int32_t k = 0; k < H; ++k)
                    o[k] += y[k];
            }
            for (int32_t kk = 0; kk < K; ++kk) {
                int32_t e = idx[t * K + kk];
                if (e < 0 || e >= E) {
                    bad = 1;
                    break;
                }
                int64_t n13 = 2LL * I * H, n2 = (int64_t)H * I;
                const float *e13s = NULL, *e2s = NULL;
                if (w_dtype == OR_E4M3) {
                    e13s = w13_s + e * (n13 / (128 * 128));
                    e2s = w2_s + e * (n2 / (128 * 128));
                }
                ffn_row(H, I, xr, expert_base(w13, w_dtype, e, n13), e13s,
                        expert_base(w2, w_dtype, e, n2), e2s, w_dtype, quant_act, h, y);
                for (int32_t k = 0; k < H; ++k)
                    o[k] += w[t * K + kk] * y[k];
            }
        }
        free(xr); free(y); free(h);
    }
    return bad;
}

/* Expert FFN on listed (token, expert) pairs: out[n] = FFN_{experts[n]}(x_t)
 * with t = tokens[n]; experts[n] == -1 selects the shared expert (R5).  This
 * is the row that the expert-sorted layout holds for that pair ([Co-design]
 * 2.3: the sorted tokens are x[order // top_k]).  out is [n, H]. */
int oracle_ffn(const oracle_cfg *c, int64_t n, const int64_t *tokens, const int32_t *experts,
               const void *x, int32_t x_dtype, const void *w13, const float *w13_s,
               const void *w2, const float *w2_s, const void *ws13, const float *ws13_s,
               const void *ws2, const float *ws2_s, int32_t w_dtype, int32_t quant_act,
               double *out)
{
    const int32_t H = c->H, I = c->I, Is = c->Is, E = c->E;
    int bad = 0;
    int32_t nmax = I > Is ? I : Is;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n; ++r) {
        int64_t t = tokens[r];
        int32_t e = experts[r];
        double *xr = malloc(sizeof(double) * H);
        double *h = malloc(sizeof(double) * (nmax > 0 ? nmax : 1));
        if (!xr || !h || e < -1 || e >= E || (e == -1 && Is == 0)) {
            bad = 1;
        } else {
            for (int32_t k = 0; k < H; ++k)
                xr[k] = mat_at(x, NULL, x_dtype, H, t, k);
            if (quant_act)
                quant_dequant_row(xr, H, quant_act);
            if (e < 0) {
                ffn_row(H, Is, xr, ws13, ws13_s, ws2, ws2_s, w_dtype, quant_act, h, out + r * H);
            } else {
                int64_t n13 = 2LL * I * H, n2 = (int64_t)H * I;
                const float *e13s = NULL, *e2s = NULL;
                if (w_dtype == OR_E4M3) {
                    e13s = w13_s + e * (n13 / (128 * 128));
                    e2s = w2_s + e * (n2 / (128 * 128));
                }
                ffn_row(H, I, xr, expert_base(w13, w_dtype, e, n13), e13s,
                        expert_base(w2, w_dtype, e, n2), e2s, w_dtype, quant_act, h, out + r * H);
            }
        }
        free(xr); free(h);
    }
    return bad;
}

/* Step 13 from expert rows in the sorted order ([Co-design] 2.3, results
 * collected back to their tokens; R6):
 *   out[t] = ys[t] + sum_k w[t,k] * y[pos[t*K + k]]
 * y is [T*K, H], ys [T, H] or NULL (no shared expert), out [T, H]. */
void oracle_combine(int64_t T, int32_t K, int32_t H, const double *y, const double *ys,
                    const int32_t *pos, const double *w, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t m = 0; m < H; ++m) {
            double acc = ys ? ys[t * H + m] : 0.0;
            for (int32_t k = 0; k < K; ++k)
                acc += w[t * K + k] * y[(int64_t)pos[t * K + k] * H + m];
            out[t * H + m] = acc;
        }
    }
}

/* ---- selection-bias update ---------------------------------------------- */

/* One load-balancing update of the selection bias (R11).  counts[e] is the
 * number of rows routed to expert e over the batch (or batches) being
 * balanced; the mean load is sum(counts) / E.  For every expert:
 *   counts[e] < mean:  bias += gamma
 *   counts[e] > mean:  bias -= gamma
 *   otherwise:         bias unchanged (bit for bit)
 * gamma is an fp32 value; the new value is computed in double (exact for
 * the sum of two fp32 values) and rounded once to fp32.  bias_in and
 * bias_out may alias.  Returns 1 for a negative or non-finite gamma, E < 1 or
 * a negative count. */
int oracle_bias_update(int32_t E, const int32_t *counts, float gamma, const float *bias_in,
                       float *bias_out)
{
    if (E < 1 || !(gamma >= 0.0f) || isinf(gamma))
        return 1;
    double total = 0.0;
    for (int32_t e = 0; e < E; ++e) {
        if (counts[e] < 0)
            return 1;
        total += counts[e];
    }
    double mean = total / E;
    for (int32_t e = 0; e < E; ++e) {
        double b = bias_in[e];
        if (counts[e] < mean)
            bias_out[e] = (float)(b + (double)gamma);
        else if (counts[e] > mean)
            bias_out[e] = (float)(b - (double)gamma);
        else
            bias_out[e] = bias_in[e];
    }
    return 0;
}

/* ---- expert FFN backward (training) ------------------------------------ */

/* Backward of one SwiGLU expert (R5) over n rows, in double.  Row r has the
 * input x_r = x[tokens[r]] and the output gradient dy_r = dy[r*H .. +H).
 * With [g; u] = W13 x, h = silu(g) u, y = W2 h, the exact derivatives are
 *   dh   = W2^T dy                 dh_i = sum_m dy_m W2[m][i]
 *   dg   = dh u silu'(g),          silu'(g) = s (1 + g (1 - s)), s = 1/(1+e^-g)
 *   du   = dh silu(g)
 *   dx_r = W13^T [dg; du]          dx_k = sum_i dg_i W13[i][k] + du_i W13[n+i][k]
 *   dW2  = sum_r dy_r h_r^T        [H, n]
 *   dW13 = sum_r [dg; du]_r x_r^T  [2n, H]
 * e is the expert (-1: the shared expert, width Is).  Outputs (any may be
 * NULL): dx [n, H], dw13 [2 n_e, H], dw2 [H, n_e], n_e = I or Is.  Weights
 * are fp32 or bf16.  Returns 1 for a bad expert, dtype or allocation. */
int oracle_ffn_backward(const oracle_cfg *c, int32_t e, int64_t n, const int64_t *tokens,
                        const void *x, int32_t x_dtype, const double *dy, const void *w13,
                        const void *w2, const void *ws13, const void *ws2, int32_t w_dtype,
                        double *dx, double *dw13, double *dw2)
{
    const int32_t H = c->H, E = c->E;
    if (e < -1 || e >= E || (e == -1 && c->Is == 0) || w_dtype == OR_E4M3)
        return 1;
    const int32_t ne = e < 0 ? c->Is : c->I;
    const void *W13 = e < 0 ? ws13 : expert_base(w13, w_dtype, e, (int64_t)2 * ne * H);
    const void *W2 = e < 0 ? ws2 : expert_base(w2, w_dtype, e, (int64_t)H * ne);
    double *xs = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * H);
    double *g = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * ne);
    double *u = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * ne);
    double *h = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * ne);
    double *da = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * 2 * ne);
    if (!xs || !g || !u || !h || !da) {
        free(xs); free(g); free(u); free(h); free(da);
        return 1;
    }
    /* forward quantities and the row gradients */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        double *xr = xs + r * H;
        for (int32_t k = 0; k < H; ++k)
            xr[k] = mat_at(x, NULL, x_dtype, H, tokens[r], k);
        for (int32_t i = 0; i < ne; ++i) {
            double gs = 0.0, us = 0.0;
            for (int32_t k = 0; k < H; ++k) {
                gs += mat_at(W13, NULL, w_dtype, H, i, k) * xr[k];
                us += mat_at(W13, NULL, w_dtype, H, ne + i, k) * xr[k];
            }
            g[r * ne + i] = gs;
            u[r * ne + i] = us;
            double sg = 1.0 / (1.0 + exp(-gs));
            h[r * ne + i] = gs * sg * us;
            double dh = 0.0;
            for (int32_t m = 0; m < H; ++m)
                dh += dy[r * H + m] * mat_at(W2, NULL, w_dtype, ne, m, i);
            da[r * 2 * ne + i] = dh * us * sg * (1.0 + gs * (1.0 - sg));
            da[r * 2 * ne + ne + i] = dh * gs * sg;
        }
        if (dx) {
            for (int32_t k = 0; k < H; ++k) {
                double acc = 0.0;
                for (int32_t q = 0; q < 2 * ne; ++q)
                    acc += da[r * 2 * ne + q] * mat_at(W13, NULL, w_dtype, H, q, k);
                dx[r * H + k] = acc;
            }
        }
    }
    if (dw2) {
#pragma omp parallel for schedule(static)
        for (int32_t m = 0; m < H; ++m)
            for (int32_t i = 0; i < ne; ++i) {
                double acc = 0.0;
                for (int64_t r = 0; r < n; ++r)
                    acc += dy[r * H + m] * h[r * ne + i];
                dw2[(int64_t)m * ne + i] = acc;
            }
    }
    if (dw13) {
#pragma omp parallel for schedule(static)
        for (int32_t q = 0; q < 2 * ne; ++q)
            for (int32_t k = 0; k < H; ++k) {
                double acc = 0.0;
                for (int64_t r = 0; r < n; ++r)
                    acc += da[r * 2 * ne + q] * xs[r * H + k];
                dw13[(int64_t)q * H + k] = acc;
            }
    }
    free(xs); free(g); free(u); free(h); free(da);
    return 0;
}

/* Quantise then dequantise, in place, each column of v [n, F] (row stride
 * F) in tiles of 128 consecutive rows from row 0 (the last tile may be
 * shorter), with the scale rule of `mode`: the column-tile form of the 1x128
 * quantiser used by the FP8 weight gradients (R15).  A short tile is
 * quantised as a 128-long tile padded with zeros, which changes neither its
 * maximum nor its codes. */
static void quant_dequant_cols(double *v, int64_t n, int32_t F, int32_t mode)
{
#pragma omp parallel for schedule(static)
    for (int32_t f = 0; f < F; ++f) {
        float tmp[128];
        uint8_t q[128];
        float sc;
        for (int64_t r0 = 0; r0 < n; r0 += 128) {
            int64_t len = n - r0 < 128 ? n - r0 : 128;
            for (int j = 0; j < 128; ++j)
                tmp[j] = j < len ? (float)v[(r0 + j) * F + f] : 0.0f;
            if (mode == OR_QUANT_POW2)
                oracle_quant_rows_pow2(1, 128, tmp, q, &sc);
            else
                oracle_quant_rows(1, 128, tmp, q, &sc);
            for (int64_t j = 0; j < len; ++j)
                v[(r0 + j) * F + f] = oracle_e4m3_decode(q[j]) * (double)sc;
        }
    }
}

/* The FP8 backward of one SwiGLU expert (R15) over the rows with inputs
 * x[tokens[r]] and output gradients dy [n, H], in the order given (the
 * expert's rows in sorted order: the column tiles of the weight gradients
 * start at the first of them).  Q_k quantises each row in 1x128 tiles
 * along its k elements (R7 or R14 by `mode`), Qc each column in tiles of
 * 128 rows, and W are the dequantised e4m3 weights (code x 128x128 block
 * scale):
 *   [g; u] = W13 Q_H(x_r),  h = silu(g) u             (the F2 forward)
 *   dh     = W2^T Q_H(dy_r)                           (contraction over H)
 *   dg     = dh u silu'(g),  du = dh silu(g)
 *   dx_r   = W13^T Q_2n([dg; du]_r)                   (contraction over 2n)
 *   dW2    = sum_r Qc(dy)_r Qc(h)_r^T                 [H, n]
 *   dW13   = sum_r Qc([dg; du])_r Qc(x)_r^T           [2n, H]
 * with every sum in double.  mode OR_QUANT_NONE gives the exact backward of
 * the dequantised weights.  w13 [E, 2I, H] with scales [E, 2I/128, H/128],
 * w2 [E, H, I] with [E, H/128, I/128]; the shared expert's likewise.  e: the
 * expert (-1: shared).  Returns 1 for a bad expert or shape, or allocation. */
int oracle_ffn_backward_fp8(const oracle_cfg *c, int32_t e, int64_t n, const int64_t *tokens,
                            const void *x, int32_t x_dtype, const double *dy,
                            const uint8_t *w13, const float *w13_s, const uint8_t *w2,
                            const float *w2_s, const uint8_t *ws13, const float *ws13_s,
                            const uint8_t *ws2, const float *ws2_s, int32_t mode, double *dx,
                            double *dw13, double *dw2)
{
    const int32_t H = c->H, E = c->E;
    if (e < -1 || e >= E || (e == -1 && c->Is == 0))
        return 1;
    const int32_t ne = e < 0 ? c->Is : c->I;
    if (H % 128 || ne % 128)
        return 1;
    const int64_t eb13 = (int64_t)(2 * ne / 128) * (H / 128), eb2 = (int64_t)(H / 128) * (ne / 128);
    const uint8_t *W13 = e < 0 ? ws13 : w13 + (int64_t)e * 2 * ne * H;
    const float *S13 = e < 0 ? ws13_s : w13_s + e * eb13;
    const uint8_t *W2 = e < 0 ? ws2 : w2 + (int64_t)e * H * ne;
    const float *S2 = e < 0 ? ws2_s : w2_s + e * eb2;
    const size_t nn = (size_t)(n > 0 ? n : 1);
    double *xs = malloc(sizeof(double) * nn * H);
    double *xq = malloc(sizeof(double) * nn * H);
    double *dyq = malloc(sizeof(double) * nn * H);
    double *h = malloc(sizeof(double) * nn * ne);
    double *da = malloc(sizeof(double) * nn * 2 * ne);
    double *daq = malloc(sizeof(double) * nn * 2 * ne);
    if (!xs || !xq || !dyq || !h || !da || !daq) {
        free(xs); free(xq); free(dyq); free(h); free(da); free(daq);
        return 1;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        double *xr = xs + r * H, *xqr = xq + r * H, *dr = dyq + r * H;
        for (int32_t k = 0; k < H; ++k) {
            xr[k] = mat_at(x, NULL, x_dtype, H, tokens[r], k);
            xqr[k] = xr[k];
            dr[k] = dy[r * H + k];
        }
        if (mode) {
            quant_dequant_row(xqr, H, mode);
            quant_dequant_row(dr, H, mode);
        }
        double *dar = da + r * 2 * ne;
        for (int32_t i = 0; i < ne; ++i) {
            double gs = 0.0, us = 0.0, dh = 0.0;
            for (int32_t k = 0; k < H; ++k) {
                gs += mat_at(W13, S13, OR_E4M3, H, i, k) * xqr[k];
                us += mat_at(W13, S13, OR_E4M3, H, ne + i, k) * xqr[k];
            }
            for (int32_t m = 0; m < H; ++m)
                dh += dr[m] * mat_at(W2, S2, OR_E4M3, ne, m, i);
            double sg = 1.0 / (1.0 + exp(-gs));
            h[r * ne + i] = gs * sg * us;
            dar[i] = dh * us * sg * (1.0 + gs * (1.0 - sg));
            dar[ne + i] = dh * gs * sg;
        }
        double *daqr = daq + r * 2 * ne;
        memcpy(daqr, dar, sizeof(double) * 2 * ne);
        if (mode)
            quant_dequant_row(daqr, 2 * ne, mode);
        if (dx) {
            for (int32_t k = 0; k < H; ++k) {
                double acc = 0.0;
                for (int32_t q = 0; q < 2 * ne; ++q)
                    acc += daqr[q] * mat_at(W13, S13, OR_E4M3, H, q, k);
                dx[r * H + k] = acc;
            }
        }
    }
    /* the weight gradients: column tiles of 128 rows (dy, h, [dg; du], x) */
    if (dw2 || dw13) {
        memcpy(dyq, dy, sizeof(double) * (size_t)n * H);   /* dyq now holds Qc(dy) */
        if (mode) {
            quant_dequant_cols(dyq, n, H, mode);
            quant_dequant_cols(h, n, ne, mode);
            quant_dequant_cols(da, n, 2 * ne, mode);
            quant_dequant_cols(xs, n, H, mode);
        }
    }
    if (dw2) {
#pragma omp parallel for schedule(static)
        for (int32_t m = 0; m < H; ++m)
            for (int32_t i = 0; i < ne; ++i) {
                double acc = 0.0;
                for (int64_t r = 0; r < n; ++r)
                    acc += dyq[r * H + m] * h[r * ne + i];
                dw2[(int64_t)m * ne + i] = acc;
            }
    }
    if (dw13) {
#pragma omp parallel for schedule(static)
        for (int32_t q = 0; q < 2 * ne; ++q)
            for (int32_t k = 0; k < H; ++k) {
                double acc = 0.0;
                for (int64_t r = 0; r < n; ++r)
                    acc += da[r * 2 * ne + q] * xs[r * H + k];
                dw13[(int64_t)q * H + k] = acc;
            }
    }
    free(xs); free(xq); free(dyq); free(h); free(da); free(daq);
    return 0;
}

/* Selected entries of the same weight gradients, one by one, for rows too
 * many for the full matrices (each entry costs O(n H)).  Entry q is
 * dW13[rr[q]][cc[q]] when which[q] == 0 and dW2[rr[q]][cc[q]] when
 * which[q] == 1, with the definitions of oracle_ffn_backward:
 *   dW13[i][k]      = sum_r dg_r[i] x_r[k],  dW13[n+i][k] = sum_r du_r[i] x_r[k]
 *   dW2[m][i]       = sum_r dy_r[m] h_r[i]
 * where g_r[i], u_r[i] and dh_r[i] are recomputed for the entry's column i. */
int oracle_ffn_backward_entries(const oracle_cfg *c, int32_t e, int64_t n, const int64_t *tokens,
                                const void *x, int32_t x_dtype, const double *dy, const void *w13,
                                const void *w2, const void *ws13, const void *ws2,
                                int32_t w_dtype, int64_t nq, const int32_t *which,
                                const int32_t *rr, const int32_t *cc, double *out)
{
    const int32_t H = c->H, E = c->E;
    if (e < -1 || e >= E || (e == -1 && c->Is == 0) || w_dtype == OR_E4M3)
        return 1;
    const int32_t ne = e < 0 ? c->Is : c->I;
    const void *W13 = e < 0 ? ws13 : expert_base(w13, w_dtype, e, (int64_t)2 * ne * H);
    const void *W2 = e < 0 ? ws2 : expert_base(w2, w_dtype, e, (int64_t)H * ne);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t q = 0; q < nq; ++q) {
        const int32_t r0 = rr[q], c0 = cc[q];
        const int dw13 = which[q] == 0;
        if ((dw13 && (r0 < 0 || r0 >= 2 * ne || c0 < 0 || c0 >= H)) ||
            (!dw13 && (r0 < 0 || r0 >= H || c0 < 0 || c0 >= ne))) {
            bad = 1;
            continue;
        }
        const int32_t i = dw13 ? r0 % ne : c0;     /* the FFN column involved */
        double acc = 0.0;
        for (int64_t r = 0; r < n; ++r) {
            double gs = 0.0, us = 0.0, dh = 0.0;
            for (int32_t k = 0; k < H; ++k) {
                double xv = mat_at(x, NULL, x_dtype, H, tokens[r], k);
                gs += mat_at(W13, NULL, w_dtype, H, i, k) * xv;
                us += mat_at(W13, NULL, w_dtype, H, ne + i, k) * xv;
            }
            double sg = 1.0 / (1.0 + exp(-gs));
            if (dw13) {
                for (int32_t m = 0; m < H; ++m)
                    dh += dy[r * H + m] * mat_at(W2, NULL, w_dtype, ne, m, i);
                double d = r0 < ne ? dh * us * sg * (1.0 + gs * (1.0 - sg)) : dh * gs * sg;
                acc += d * mat_at(x, NULL, x_dtype, H, tokens[r], c0);
            } else {
                acc += dy[r * H + r0] * (gs * sg * us);
            }
        }
        out[q] = acc;
    }
    return bad;
}
