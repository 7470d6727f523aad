/* prefill_oracle.h — plain CPU oracle for the batched int8-weight prefill path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this code; only the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no source, header, table or constant with
 * the HIP library (include/libprefill.h and int8_weight_gemm_amd/csrc).
 *
 * Everything is per token: no chunking, blocking or batching.  Whatever the GPU
 * path computes in chunks must equal these per-token results byte for byte.
 * All pointers are host pointers, owned by the caller.  Arrays are row-major.
 *
 * Sources (the web pages on the subject):
 *   [cellm] "Batched Prefill" (jeffasante.github.io/cellm), sections
 *           The Problem, The arithmetic, The Solution, What Stays Sequential,
 *           Correctness.
 *   [sip]   "Single-pass prefill" (SipLLM docs), section "The fix".
 *   [red]   "Red Lite dev24 — prefill: pre-gated expert prefetch and parallel
 *           routing", sections "What changed" and "Scope boundary".
 * Where the pages leave an arithmetic detail open (quantiser rounding, epilogue
 * association, stack dataflow, softmax exp) the reading taken is written next to
 * the function that implements it.
 */
#ifndef PREFILL_ORACLE_H
#define PREFILL_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes: 0 ok, -1 bad argument, -2 non-finite input value. */

/* The nonlinearity between the gate/up products and the down product.
 * OR_ACT_NONE: the reading used when the pages name no activation (the stack's
 * down reads quantise(up); an expert's down reads quantise(g * u)).
 * OR_ACT_SWIGLU: the gated SiLU of the feed-forward blocks of the model
 * families the pages run (the pages name gate, up and down projections but no
 * formula): r_i = fl(silu(g_i) * u_i) with silu(g) = fl(g / fl(1 + expf_cr(-g))),
 * the stack's down reading quantise(r) (gate then feeds it) and an expert's
 * down reading quantise(r). */
#define OR_ACT_NONE 0
#define OR_ACT_SWIGLU 1

/* Per-token symmetric quantisation, once per token row [cellm §The Solution:
 * activations quantised once per batch]: amax = max|x_k| (exact),
 * s = fl(amax / 127), q_k = clamp(roundf(fl(x_k / s)), -127, 127) with roundf
 * rounding halves away from zero; s == 0 gives q = 0.  x [M][K] -> q [M][K],
 * s [M]. */
int or_quantize(const float* x, int64_t M, int64_t K, int8_t* q, float* s);

/* One int8 GEMV, the per-token product of [cellm §The Problem]:
 * acc_n = sum_k W[n][k] * q[k] in exact int32, then
 * y[n] = fl( fl((float)acc_n) * fl(w_scale[n] * a_scale) ).  W [N][K]. */
int or_gemv(const int8_t* W, const float* w_scale, int64_t N, int64_t K,
            const int8_t* q, float a_scale, float* y);

/* or_gemv applied to each of M token rows in turn (no GEMM of its own:
 * [cellm §Correctness] requires the batched product to equal per-token GEMVs
 * byte for byte).  q [M][K], a_scale [M] -> y [M][N] token-major. */
int or_linear_per_token(const int8_t* W, const float* w_scale, int64_t N, int64_t K,
                        const int8_t* q, const float* a_scale, int64_t M, float* y,
                        int threads);

/* The projection stack swept token by token [sip "The fix"; cellm §The Solution].
 * Per layer l, with h the layer input (h = x for l = 0):
 *   (a, sa) = quantise(h);  p_j = gemv(W[l][j], a, sa) for j = q,k,v,o,gate,up;
 *   (b, sb) = quantise(up); down = gemv(W[l][6], b, sb);  next h = down.
 * With act = OR_ACT_SWIGLU, (b, sb) = quantise(silu(gate) * up) instead.
 * Weights: W[l*7 + j], w_scale[l*7 + j]; shapes q,k,v,o [H][H], gate,up [F][H],
 * down [H][F].  x [P][H] -> y [P][H].  proj, when not NULL, receives every
 * projection output: proj[((l*P + t) * (5H + 2F)) + off_j + n] with the seven
 * outputs concatenated in the order q,k,v,o,gate,up,down. */
int or_stack(int64_t L, int64_t H, int64_t F, const int8_t* const* W,
             const float* const* w_scale, const float* x, int64_t P, float* y,
             float* proj, int threads, int act);

/* The stack with causal attention over the prompt (n_heads heads of
 * d = H / n_heads values) [cellm §What Stays Sequential: attention runs per
 * position; sip "The fix": position t attends over the K/V history
 * kv_[layer][0..t]].  Per layer, each token's q, k, v, gate, up come from
 * quantise(h); k and v are written to the cache kv [L][2][P][H] (k at [l][0],
 * v at [l][1]); the token's attention over positions 0..t of its layer
 * (per head: f32 scores in ascending index with c = fl(1/fl(sqrt(d))), softmax
 * with expf_cr and an ascending sum, the probability-weighted sum of v rows in
 * ascending position) is quantised and feeds o; down as in or_stack.  y, proj as
 * in or_stack. */
int or_stack_attn(int64_t L, int64_t H, int64_t F, int64_t n_heads, const int8_t* const* W,
                  const float* const* w_scale, const float* x, int64_t P, float* y,
                  float* proj, float* kv, int threads, int act);

/* Correctly rounded binary32 exp (the exact exponential rounded to nearest,
 * ties to even).  Aborts if the long-double evaluation cannot decide the
 * rounding (never observed on the domain used; checked exhaustively by the
 * tests). */
float or_expf_cr(float x);
int or_expf_cr_array(const float* x, int64_t n, float* y, int threads);

/* silu(g) = fl(g / fl(1 + or_expf_cr(-g))), each operation rounded on its own. */
float or_silu(float g);

/* Router logits of one token, the f32 product of [red "What changed", item 1]:
 * l[e] = 0, then for k ascending l[e] = fl(l[e] + fl(Wr[e][k] * x[k])). */
int or_router(const float* Wr, int64_t E, int64_t H, const float* x, float* logits);

/* Softmax over E logits, then the top_k largest probabilities [red "What
 * changed", item 2]: m = max l; z_e = expf_cr(fl(l_e - m)); S = sum of z in
 * ascending e; p_e = fl(z_e / S).  ids ordered by descending p, ties to the
 * lower id; weights[j] = p[ids[j]] (not renormalised).  With renorm = 1 the
 * weights are renormalised over the chosen experts: T = sum of weights[j] in
 * rank order j = 0 .. top_k-1, then weights[j] = fl(weights[j] / T). */
int or_softmax_topk(const float* logits, int64_t E, int64_t top_k,
                    int32_t* ids, float* weights, int renorm);

/* One expert applied to one token: g = gemv(Wg_e, xq), u = gemv(Wu_e, xq),
 * r_i = fl(g_i * u_i) (act OR_ACT_NONE) or fl(silu(g_i) * u_i) (OR_ACT_SWIGLU),
 * (hq, hs) = quantise(r), y = gemv(Wd_e, hq, hs).
 * Wg, Wu [E][I][H]; Wd [E][H][I]; sg, su [E][I]; sd [E][H]. */
int or_expert(int64_t H, int64_t I, const int8_t* Wg, const int8_t* Wu,
              const int8_t* Wd, const float* sg, const float* su, const float* sd,
              int64_t e, const int8_t* xq, float xs, float* y, int act);

/* Mixture-of-experts prefill of T tokens, token by token:
 * xq = quantise(x_t); logits = router(x_t); (ids, w) = softmax_topk(logits);
 * out_t = +0, then for each selected expert in ascending id
 * out_t[j] = fl(out_t[j] + fl(w_e * y_e[j])).  ids, weights [T][top_k].
 * act and renorm select the variants of or_expert and or_softmax_topk. */
int or_moe(int64_t E, int64_t top_k, int64_t H, int64_t I, const float* Wr,
           const int8_t* Wg, const int8_t* Wu, const int8_t* Wd,
           const float* sg, const float* su, const float* sd,
           const float* x, int64_t T, int32_t* ids, float* weights, float* out,
           int threads, int act, int renorm);

#ifdef __cplusplus
}
#endif
#endif
