/* prefill_oracle.c — plain, slow, per-token CPU oracle (C11 + libm + OpenMP).
 *
 * TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  The HIP product path never includes,
 * links or calls it, and it includes nothing from the product.
 *
 * Build: gcc -std=c11 -O2 -ftree-vectorize -mavx2 -ffp-contract=off -fopenmp
 *        -fPIC -shared (no fast-math: every float operation below is one IEEE
 *        binary32 operation rounded to nearest even, in the written order).
 *
 * Sources and readings: see prefill_oracle.h.  Every function here is the plain
 * definition; OpenMP only spreads independent tokens over threads.
 */
#include "prefill_oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* Quantise one token row.  Reading of the per-batch activation quantisation
 * ("Batched Prefill", §The Solution): symmetric, scale s = absmax/127, values
 * divided by s (IEEE division) and rounded half away from zero (C roundf),
 * clamped to [-127, 127]; an all-zero row gets s = 0 and q = 0. */
static int quantize_row(const float* x, int64_t K, int8_t* q, float* s_out)
{
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        if (!isfinite(x[k])) return -2;
        float a = fabsf(x[k]);
        if (a > amax) amax = a;
    }
    float s = amax / 127.0f;
    *s_out = s;
    if (s == 0.0f) {
        memset(q, 0, (size_t)K);
        return 0;
    }
    for (int64_t k = 0; k < K; ++k) {
        float v = x[k] / s;
        float r = roundf(v);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[k] = (int8_t)r;
    }
    return 0;
}

int or_quantize(const float* x, int64_t M, int64_t K, int8_t* q, float* s)
{
    if (!x || !q || !s || M < 0 || K <= 0) return -1;
    for (int64_t t = 0; t < M; ++t) {
        int rc = quantize_row(x + t * K, K, q + t * K, s + t);
        if (rc) return rc;
    }
    return 0;
}

/* The per-token product ("Batched Prefill", §The Problem: one GEMV per token).
 * The int32 sum is exact (|acc| <= K * 127 * 127 < 2^31 for K <= 131072), so the
 * order of the k loop is immaterial; the epilogue is (float)acc * (ws * as). */
static void gemv_row_block(const int8_t* W, const float* w_scale, int64_t N, int64_t K,
                           const int8_t* q, float a_scale, float* y)
{
    for (int64_t n = 0; n < N; ++n) {
        const int8_t* w = W + n * K;
        int32_t acc = 0;
        for (int64_t k = 0; k < K; ++k) acc += (int32_t)w[k] * (int32_t)q[k];
        float scale = w_scale[n] * a_scale;
        y[n] = (float)acc * scale;
    }
}

int or_gemv(const int8_t* W, const float* w_scale, int64_t N, int64_t K,
            const int8_t* q, float a_scale, float* y)
{
    if (!W || !w_scale || !q || !y || N <= 0 || K <= 0 || K > 131072) return -1;
    gemv_row_block(W, w_scale, N, K, q, a_scale, y);
    return 0;
}

int or_linear_per_token(const int8_t* W, const float* w_scale, int64_t N, int64_t K,
                        const int8_t* q, const float* a_scale, int64_t M, float* y,
                        int threads)
{
    if (!W || !w_scale || !q || !a_scale || !y || N <= 0 || K <= 0 || M < 0 || K > 131072)
        return -1;
    if (threads < 1) threads = 1;
#pragma omp parallel for num_threads(threads) schedule(dynamic, 1)
    for (int64_t t = 0; t < M; ++t)
        gemv_row_block(W, w_scale, N, K, q + t * K, a_scale[t], y + t * N);
    return 0;
}

/* The stack, one token at a time ("Single-pass prefill", "The fix": every
 * position goes through every layer; per-position work is the same as the
 * per-token path).  Dataflow inside a layer (a reading: the pages batch only the
 * linear projections, and the sequential attention that would sit between them
 * is not part of this path): all six K = H projections read quantise(h); down
 * reads quantise(up); the next layer's input is down, unchanged. */
int or_stack(int64_t L, int64_t H, int64_t F, const int8_t* const* W,
             const float* const* w_scale, const float* x, int64_t P, float* y,
             float* proj, int threads, int act)
{
    if (act != OR_ACT_NONE && act != OR_ACT_SWIGLU) return -1;
    if (!W || !w_scale || !x || !y || L <= 0 || H <= 0 || F <= 0 || P < 0) return -1;
    if (H > 131072 || F > 131072) return -1;
    for (int64_t i = 0; i < 7 * L; ++i)
        if (!W[i] || !w_scale[i]) return -1;
    if (threads < 1) threads = 1;
    const int64_t nrow[7] = {H, H, H, H, F, F, H};
    int64_t off[8];
    off[0] = 0;
    for (int j = 0; j < 7; ++j) off[j + 1] = off[j] + nrow[j];
    const int64_t total = off[7];
    int status = 0;

#pragma omp parallel num_threads(threads)
    {
        float* h = (float*)malloc(sizeof(float) * (size_t)H);
        float* outs = (float*)malloc(sizeof(float) * (size_t)total);
        float* r = (float*)malloc(sizeof(float) * (size_t)F);
        int8_t* a = (int8_t*)malloc((size_t)(F > H ? F : H));
        int failed = (!h || !outs || !r || !a);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < P; ++t) {
            if (failed) continue;
            memcpy(h, x + t * H, sizeof(float) * (size_t)H);
            for (int64_t l = 0; l < L && !failed; ++l) {
                float sa;
                if (quantize_row(h, H, a, &sa)) { failed = 1; break; }
                for (int j = 0; j < 6; ++j)
                    gemv_row_block(W[l * 7 + j], w_scale[l * 7 + j], nrow[j], H, a, sa,
                                   outs + off[j]);
                /* the down projection's input: up, or silu(gate) * up */
                const float* din = outs + off[5];
                if (act == OR_ACT_SWIGLU) {
                    for (int64_t i = 0; i < F; ++i) r[i] = or_silu(outs[off[4] + i]) * outs[off[5] + i];
                    din = r;
                }
                float sb;
                if (quantize_row(din, F, a, &sb)) { failed = 1; break; }
                gemv_row_block(W[l * 7 + 6], w_scale[l * 7 + 6], H, F, a, sb, outs + off[6]);
                if (proj)
                    memcpy(proj + (l * P + t) * total, outs, sizeof(float) * (size_t)total);
                memcpy(h, outs + off[6], sizeof(float) * (size_t)H);
            }
            if (!failed) memcpy(y + t * H, h, sizeof(float) * (size_t)H);
        }
        if (failed) {
#pragma omp atomic write
            status = -2;
        }
        free(h);
        free(outs);
        free(r);
        free(a);
    }
    return status;
}

/* Causal attention of one token over the K/V history of its layer ("Batched
 * Prefill", What Stays Sequential: attention runs per position inside each
 * chunk; "Single-pass prefill", "The fix": position t attends over
 * kv_[layer][0..t], written before it).  For head hd (d = H / n_heads values
 * from column hd*d): s_j = fl(dot(q, K[j]) * c) for j = 0..t, the dot an f32 sum
 * in ascending index of separately rounded products and c = fl(1 / fl(sqrt(d)));
 * m = max s_j; z_j = expf_cr(fl(s_j - m)); S = sum of z_j in ascending j;
 * p_j = fl(z_j / S); out[i] = sum over j ascending of fl(p_j * V[j][i]) from +0.
 * K and V point at position 0 of the layer's cache, rows of H values. */
static void attend(const float* q, const float* K, const float* V, int64_t t, int64_t H,
                   int64_t n_heads, float* z, float* out)
{
    const int64_t d = H / n_heads;
    const float c = 1.0f / sqrtf((float)d);
    for (int64_t hd = 0; hd < n_heads; ++hd) {
        const int64_t c0 = hd * d;
        float m = 0.0f;
        for (int64_t j = 0; j <= t; ++j) {
            float acc = 0.0f;
            for (int64_t i = 0; i < d; ++i) {
                float pr = q[c0 + i] * K[j * H + c0 + i];
                acc = acc + pr;
            }
            z[j] = acc * c;
            if (j == 0 || z[j] > m) m = z[j];
        }
        float S = 0.0f;
        for (int64_t j = 0; j <= t; ++j) {
            z[j] = or_expf_cr(z[j] - m);
            S = S + z[j];
        }
        for (int64_t j = 0; j <= t; ++j) z[j] = z[j] / S;
        for (int64_t i = 0; i < d; ++i) {
            float o = 0.0f;
            for (int64_t j = 0; j <= t; ++j) {
                float pr = z[j] * V[j * H + c0 + i];
                o = o + pr;
            }
            out[c0 + i] = o;
        }
    }
}

/* The stack with causal attention, swept the way "Single-pass prefill"
 * describes ("The fix"): for each layer, every prompt position goes through it
 * in order, and position t's attention reads the K/V history 0..t of that
 * layer.  Per layer and token, with h the layer input:
 *   (a, sa) = quantise(h); q, k, v, gate, up = gemv(., a, sa);
 *   kv[l][0][t] = k, kv[l][1][t] = v (the cache);
 *   att = attend(q, kv[l][0][0..t], kv[l][1][0..t]);
 *   (ao, sao) = quantise(att); o = gemv(W_o, ao, sao);
 *   (b, sb) = quantise(up) (or quantise(silu(gate) * up) with OR_ACT_SWIGLU);
 *   down = gemv(W_down, b, sb); the next layer's h = down.
 * The attention output feeds o, which, as in or_stack, feeds nothing further.
 * Tokens of one phase are independent, so each phase runs over all tokens of
 * the layer (threads over tokens) before the next. */
int or_stack_attn(int64_t L, int64_t H, int64_t F, int64_t n_heads, const int8_t* const* W,
                  const float* const* w_scale, const float* x, int64_t P, float* y,
                  float* proj, float* kv, int threads, int act)
{
    if (!W || !w_scale || !x || !y || !kv || L <= 0 || H <= 0 || F <= 0 || P < 0) return -1;
    if (H > 131072 || F > 131072 || n_heads <= 0 || H % n_heads != 0) return -1;
    if (act != OR_ACT_NONE && act != OR_ACT_SWIGLU) return -1;
    for (int64_t i = 0; i < 7 * L; ++i)
        if (!W[i] || !w_scale[i]) return -1;
    if (threads < 1) threads = 1;
    const int64_t nrow[7] = {H, H, H, H, F, F, H};
    int64_t off[8];
    off[0] = 0;
    for (int j = 0; j < 7; ++j) off[j + 1] = off[j] + nrow[j];
    const int64_t total = off[7];
    float* h = (float*)malloc(sizeof(float) * (size_t)(P * H + 1));
    float* outs = (float*)malloc(sizeof(float) * (size_t)(P * total + 1));
    if (!h || !outs) { free(h); free(outs); return -1; }
    memcpy(h, x, sizeof(float) * (size_t)(P * H));
    int status = 0;
    for (int64_t l = 0; l < L && !status; ++l) {
        float* Kc = kv + (l * 2 + 0) * P * H;
        float* Vc = kv + (l * 2 + 1) * P * H;
        /* projections from quantise(h) (o comes after the attention) */
#pragma omp parallel for num_threads(threads) schedule(dynamic, 1)
        for (int64_t t = 0; t < P; ++t) {
            int8_t* a = (int8_t*)malloc((size_t)H);
            float sa;
            if (!a || quantize_row(h + t * H, H, a, &sa)) {
#pragma omp atomic write
                status = -2;
                free(a);
                continue;
            }
            float* ot = outs + t * total;
            const int js[5] = {0, 1, 2, 4, 5};
            for (int u = 0; u < 5; ++u) {
                const int j = js[u];
                gemv_row_block(W[l * 7 + j], w_scale[l * 7 + j], nrow[j], H, a, sa, ot + off[j]);
            }
            memcpy(Kc + t * H, ot + off[1], sizeof(float) * (size_t)H);
            memcpy(Vc + t * H, ot + off[2], sizeof(float) * (size_t)H);
            free(a);
        }
        if (status) break;
        /* attention over positions 0..t, then o; the gated input of down; down */
#pragma omp parallel for num_threads(threads) schedule(dynamic, 1)
        for (int64_t t = 0; t < P; ++t) {
            float* z = (float*)malloc(sizeof(float) * (size_t)(P + 1));
            float* att = (float*)malloc(sizeof(float) * (size_t)H);
            float* r = (float*)malloc(sizeof(float) * (size_t)F);
            int8_t* a = (int8_t*)malloc((size_t)(F > H ? F : H));
            float* ot = outs + t * total;
            int bad = (!z || !att || !r || !a);
            if (!bad) {
                attend(ot + off[0], Kc, Vc, t, H, n_heads, z, att);
                float so;
                bad = quantize_row(att, H, a, &so) != 0;
                if (!bad) gemv_row_block(W[l * 7 + 3], w_scale[l * 7 + 3], H, H, a, so, ot + off[3]);
            }
            if (!bad) {
                const float* din = ot + off[5];
                if (act == OR_ACT_SWIGLU) {
                    for (int64_t i = 0; i < F; ++i) r[i] = or_silu(ot[off[4] + i]) * ot[off[5] + i];
                    din = r;
                }
                float sb;
                bad = quantize_row(din, F, a, &sb) != 0;
                if (!bad) gemv_row_block(W[l * 7 + 6], w_scale[l * 7 + 6], H, F, a, sb, ot + off[6]);
            }
            if (bad) {
#pragma omp atomic write
                status = -2;
            } else {
                if (proj) memcpy(proj + (l * P + t) * total, ot, sizeof(float) * (size_t)total);
                memcpy(h + t * H, ot + off[6], sizeof(float) * (size_t)H);
            }
            free(z); free(att); free(r); free(a);
        }
    }
    if (!status) memcpy(y, h, sizeof(float) * (size_t)(P * H));
    free(h);
    free(outs);
    return status;
}

/* Correctly rounded exp in binary32.  expl works in the x87 64-bit-significand
 * format with error below one unit of that format, i.e. about 2^-63 relative,
 * while rounding to binary32 needs to know on which side of the midpoint between
 * two neighbouring floats the exact value lies.  When the long-double value is
 * farther than 2^-58 (relative) from that midpoint, the rounding of the exact
 * value and of the long-double value agree; closer than that the oracle stops. */
float or_expf_cr(float x)
{
    if (isnan(x)) return x;
    if (x == -INFINITY) return 0.0f;
    long double y = expl((long double)x);
    float f = (float)y;
    if (isinf(f) || y == 0.0L) return f;
    float g = (y > (long double)f) ? nextafterf(f, INFINITY) : nextafterf(f, -INFINITY);
    long double mid = ((long double)f + (long double)g) * 0.5L;
    long double gap = fabsl(y - mid);
    if (gap <= fabsl(y) * 0x1p-58L) {
        fprintf(stderr, "or_expf_cr: cannot decide rounding for x = %a\n", (double)x);
        abort();
    }
    return f;
}

/* or_expf_cr over an array (threads over elements). */
int or_expf_cr_array(const float* x, int64_t n, float* y, int threads)
{
    if (!x || !y || n < 0) return -1;
    if (threads < 1) threads = 1;
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = or_expf_cr(x[i]);
    return 0;
}

/* SiLU through the correctly rounded exp, each step rounded on its own:
 * silu(g) = fl(g / fl(1 + expf_cr(-g))).  For g below about -88.7, exp(-g)
 * overflows to +inf and the quotient is -0. */
float or_silu(float g)
{
    float e = or_expf_cr(-g);
    float d = 1.0f + e;
    return g / d;
}

/* Router product for one token ("Red Lite dev24", What changed, item 1: the
 * router is one extra f32 GEMM).  The summation order the page leaves open is
 * fixed here: ascending k, each product and each sum rounded on its own. */
int or_router(const float* Wr, int64_t E, int64_t H, const float* x, float* logits)
{
    if (!Wr || !x || !logits || E <= 0 || H <= 0) return -1;
    for (int64_t e = 0; e < E; ++e) {
        const float* w = Wr + e * H;
        float acc = 0.0f;
        for (int64_t k = 0; k < H; ++k) {
            float p = w[k] * x[k];
            acc = acc + p;
        }
        logits[e] = acc;
    }
    return 0;
}

/* Softmax and top-k selection of one token ("Red Lite dev24", What changed,
 * item 2: softmax top-10 per token, ids and weights identical to the
 * single-token routine).  Readings: exp is the correctly rounded expf, the
 * normaliser sums in ascending expert id, ties in p go to the lower id, and the
 * weights are the softmax probabilities of the chosen experts. */
int or_softmax_topk(const float* logits, int64_t E, int64_t top_k,
                    int32_t* ids, float* weights, int renorm)
{
    if (!logits || !ids || !weights || E <= 0 || top_k <= 0 || top_k > E) return -1;
    if (renorm != 0 && renorm != 1) return -1;
    float* p = (float*)malloc(sizeof(float) * (size_t)E);
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    if (!p || !taken) { free(p); free(taken); return -1; }
    float m = logits[0];
    for (int64_t e = 0; e < E; ++e) {
        if (!isfinite(logits[e])) { free(p); free(taken); return -2; }
        if (logits[e] > m) m = logits[e];
    }
    float S = 0.0f;
    for (int64_t e = 0; e < E; ++e) {
        p[e] = or_expf_cr(logits[e] - m);
        S = S + p[e];
    }
    for (int64_t e = 0; e < E; ++e) p[e] = p[e] / S;
    for (int64_t j = 0; j < top_k; ++j) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || p[e] > p[best]) best = e;
        }
        taken[best] = 1;
        ids[j] = (int32_t)best;
        weights[j] = p[best];
    }
    if (renorm) {
        /* weights over the chosen experts only: T = the chosen p summed in
         * rank order (descending p, ties to the lower id), w_j = p_j / T */
        float T = 0.0f;
        for (int64_t j = 0; j < top_k; ++j) T = T + weights[j];
        for (int64_t j = 0; j < top_k; ++j) weights[j] = weights[j] / T;
    }
    free(p);
    free(taken);
    return 0;
}

/* One expert on one token.  Reading of the expert block (the page names gate,
 * up and down projections but no activation): r = g * u elementwise, quantised
 * per (token, expert) row before the down projection. */
static int expert_apply(int64_t H, int64_t I, const int8_t* Wg, const int8_t* Wu,
                        const int8_t* Wd, const float* sg, const float* su, const float* sd,
                        int64_t e, const int8_t* xq, float xs, float* y,
                        float* g, float* u, int8_t* hq, int act)
{
    gemv_row_block(Wg + e * I * H, sg + e * I, I, H, xq, xs, g);
    gemv_row_block(Wu + e * I * H, su + e * I, I, H, xq, xs, u);
    if (act == OR_ACT_SWIGLU)
        for (int64_t i = 0; i < I; ++i) g[i] = or_silu(g[i]) * u[i];
    else
        for (int64_t i = 0; i < I; ++i) g[i] = g[i] * u[i];
    float hs;
    int rc = quantize_row(g, I, hq, &hs);
    if (rc) return rc;
    gemv_row_block(Wd + e * H * I, sd + e * H, H, I, hq, hs, y);
    return 0;
}

int or_expert(int64_t H, int64_t I, const int8_t* Wg, const int8_t* Wu,
              const int8_t* Wd, const float* sg, const float* su, const float* sd,
              int64_t e, const int8_t* xq, float xs, float* y, int act)
{
    if (!Wg || !Wu || !Wd || !sg || !su || !sd || !xq || !y || H <= 0 || I <= 0 || e < 0)
        return -1;
    if (act != OR_ACT_NONE && act != OR_ACT_SWIGLU) return -1;
    float* g = (float*)malloc(sizeof(float) * (size_t)I);
    float* u = (float*)malloc(sizeof(float) * (size_t)I);
    int8_t* hq = (int8_t*)malloc((size_t)I);
    int rc = (!g || !u || !hq) ? -1
                               : expert_apply(H, I, Wg, Wu, Wd, sg, su, sd, e, xq, xs, y, g, u, hq, act);
    free(g);
    free(u);
    free(hq);
    return rc;
}

int or_moe(int64_t E, int64_t top_k, int64_t H, int64_t I, const float* Wr,
           const int8_t* Wg, const int8_t* Wu, const int8_t* Wd,
           const float* sg, const float* su, const float* sd,
           const float* x, int64_t T, int32_t* ids, float* weights, float* out,
           int threads, int act, int renorm)
{
    if (!Wr || !Wg || !Wu || !Wd || !sg || !su || !sd || !x || !ids || !weights || !out)
        return -1;
    if ((act != OR_ACT_NONE && act != OR_ACT_SWIGLU) || (renorm != 0 && renorm != 1)) return -1;
    if (E <= 0 || top_k <= 0 || top_k > E || H <= 0 || I <= 0 || T < 0) return -1;
    if (H > 131072 || I > 131072) return -1;
    if (threads < 1) threads = 1;
    int status = 0;
#pragma omp parallel num_threads(threads)
    {
        float* logits = (float*)malloc(sizeof(float) * (size_t)E);
        int8_t* xq = (int8_t*)malloc((size_t)H);
        float* y = (float*)malloc(sizeof(float) * (size_t)H);
        float* g = (float*)malloc(sizeof(float) * (size_t)I);
        float* u = (float*)malloc(sizeof(float) * (size_t)I);
        int8_t* hq = (int8_t*)malloc((size_t)I);
        unsigned char* chosen = (unsigned char*)malloc((size_t)E);
        int failed = (!logits || !xq || !y || !g || !u || !hq || !chosen) ? -1 : 0;
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            if (failed) continue;
            const float* xt = x + t * H;
            float xs;
            int rc = quantize_row(xt, H, xq, &xs);
            if (!rc) rc = or_router(Wr, E, H, xt, logits);
            if (!rc) rc = or_softmax_topk(logits, E, top_k, ids + t * top_k, weights + t * top_k, renorm);
            if (rc) { failed = rc; continue; }
            /* combine in ascending expert id */
            memset(chosen, 0, (size_t)E);
            for (int64_t j = 0; j < top_k; ++j) chosen[ids[t * top_k + j]] = 1;
            float* o = out + t * H;
            for (int64_t n = 0; n < H; ++n) o[n] = 0.0f;
            for (int64_t e = 0; e < E && !failed; ++e) {
                if (!chosen[e]) continue;
                float w = 0.0f;
                for (int64_t j = 0; j < top_k; ++j)
                    if (ids[t * top_k + j] == e) w = weights[t * top_k + j];
                rc = expert_apply(H, I, Wg, Wu, Wd, sg, su, sd, e, xq, xs, y, g, u, hq, act);
                if (rc) { failed = rc; break; }
                for (int64_t n = 0; n < H; ++n) {
                    float c = w * y[n];
                    o[n] = o[n] + c;
                }
            }
        }
        if (failed) {
#pragma omp atomic write
            status = failed;
        }
        free(logits); free(xq); free(y); free(g); free(u); free(hq); free(chosen);
    }
    return status;
}
