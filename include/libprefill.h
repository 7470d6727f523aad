/* libprefill.h — C ABI of the batched int8-weight prefill library (MI355X, gfx950).
 *
 * The problem (from the pages on the subject):
 *   "Batched Prefill" (cellm), §The Problem and §The arithmetic: running a prompt
 *   one token at a time performs one GEMV per token and re-reads every weight once
 *   per prompt token, so prefill is bound by weight traffic.
 *   Same page, §The Solution: run each linear projection as one int8 GEMM over a
 *   chunk of tokens, quantising the chunk's activations once, so each weight byte
 *   is read once per chunk and does chunk-many multiply-accumulates.
 *   Same page, §Correctness: the batched result must equal the per-token result
 *   byte for byte, and a runtime switch must select either path.
 *   "Single-pass prefill" (SipLLM), "The fix": sweep every prompt position
 *   through a layer while that layer's weights are loaded, layer after layer.
 *   "Red Lite dev24", "What changed": mixture-of-experts prefill of a 512-token
 *   chunk routes every token (softmax top-10), takes the union of the selected
 *   experts and runs the experts on their token groups.
 *
 * Conventions (all entry points):
 *   - Array arguments are DEVICE pointers owned by the caller.  int8 matrices
 *     and f32 inputs that are read with 128-bit loads (x of the quantiser, the
 *     stack and the experts; the projection buffer) are 16-byte aligned; scales,
 *     ids and f32 outputs need 4-byte alignment.
 *     Host-side descriptors (pf_stack, pf_layer, pf_moe, pf_stack_stats) are
 *     read during the call only.
 *   - Layouts are row-major.  A weight W is [N][K] (K contiguous); activations
 *     and outputs are token-major: x [M][K], y [M][N].
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream); results are ready once the stream is synchronised.  Device faults
 *     surface at that synchronisation.
 *   - Arguments are validated on the host before any device work is queued;
 *     a rejected call returns a negative status and touches nothing.
 *   - Outputs are fully overwritten, never accumulated into.
 *   - The library allocates no device memory inside calls.  Calls that need
 *     scratch memory take a caller-owned workspace whose size comes from the
 *     matching *_workspace() query; its contents on entry do not matter and
 *     are undefined on return.  Calls that share one workspace must be ordered
 *     (same stream); calls that overlap on one workspace race.
 *   - Input activations must be finite; results for NaN or Inf inputs are
 *     unspecified.
 *   - State kept across calls: a per-device architecture check and, for
 *     pf_prefill_stack, two library-owned streams per device (default
 *     priority) with their fork/join events, created on first use and kept
 *     until the process ends.  A mutex per device serialises the stack calls
 *     that use them, so concurrent stack calls from several host threads on
 *     one device run one after the other; every other entry point is
 *     reentrant.
 *   - K of every product must be a positive multiple of 64 and at most 131072,
 *     which keeps every int32 accumulator exact (131072 * 127 * 127 < 2^31).
 *   - A weight matrix (N x K) and a chunk of quantised tokens (M x K) must each
 *     hold fewer than 2^32 bytes (the product kernels address them by 32-bit
 *     offsets): pf_gemm_i8_chunk checks N * K and M * K, pf_prefill_stack
 *     hidden * ffn and chunk * max(hidden, ffn); larger ones are rejected with
 *     PF_EINVAL.
 *
 * Arithmetic (bit-exact with the plain per-token CPU definition):
 *   quantise:  amax = max_k |x_k|; s = fl(amax / 127); q_k = clamp(roundf(fl(x_k / s)),
 *              -127, 127) with roundf rounding halves away from zero; s = 0 -> q = 0.
 *   product:   acc[t][n] = sum_k W[n][k] * q[t][k] in exact int32;
 *              y[t][n] = fl( fl((float)acc) * fl(w_scale[n] * a_scale[t]) ).
 */
#ifndef LIBPREFILL_H
#define LIBPREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The entry points below are the library's only exported symbols. */
#define PF_API __attribute__((visibility("default")))

typedef int pf_status;
#define PF_OK          0
#define PF_EINVAL     -1  /* bad argument: null, size, alignment, overlap       */
#define PF_ENODEV     -2  /* no HIP device, or the current device is not gfx950 */
#define PF_ELAUNCH    -3  /* a HIP launch or runtime call failed                 */
#define PF_EWORKSPACE -4  /* workspace missing or smaller than required          */
#define PF_EINTERNAL  -5  /* unexpected internal error                           */

/* Human-readable name of a status code (static string). */
PF_API const char* pf_status_string(pf_status status);

/* Checks that a gfx950 device is current and looks up the device address of
 * pf_gemm_i8_chunk_noalloc's scratch array on it.  Every entry point checks
 * the device on first use; calling this first only moves the cost.  PF_ENODEV
 * without a device. */
PF_API pf_status pf_init(void);

/* Zero-fills `bytes` of device memory on `stream` (a fill kernel, no memset
 * node); a convenience for callers that want a defined workspace. */
PF_API pf_status pf_workspace_clear(void* workspace, size_t bytes, void* stream);

/* Per-token symmetric int8 quantisation of a chunk, done once per chunk
 * ("Batched Prefill", §The Solution: activations are quantised once per batch,
 * not once per weight row).
 * x [M][ldx] f32 (first K of each row used) -> xq [M][K] int8, a_scale [M] f32.
 * M = 0 is a no-op.  ldx >= K, ldx % 4 == 0. */
PF_API pf_status pf_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx,
                          int8_t* xq, float* a_scale, void* stream);

/* Workspace bytes pf_gemm_i8_chunk may use to split K across workgroups
 * (0 is always accepted; a larger workspace only adds parallelism). */
PF_API size_t pf_gemm_i8_chunk_workspace(int64_t N, int64_t K, int64_t M);

/* One projection over a chunk of M tokens ("Batched Prefill", §The Solution:
 * each weight row is loaded once and dotted against every token column).
 * W [N][K] int8, w_scale [N] f32, xq [M][K] int8, a_scale [M] f32 -> y [M][N]
 * f32 (token-major).  Chooses an MFMA kernel by M (skinny M <= 64, tiled above).
 * workspace may be NULL with ws_bytes 0. */
PF_API pf_status pf_gemm_i8_chunk(const int8_t* W, const float* w_scale, int64_t N, int64_t K,
                           const int8_t* xq, const float* a_scale, int64_t M, float* y,
                           void* workspace, size_t ws_bytes, void* stream);

/* pf_gemm_i8_chunk for callers that cannot allocate or pass device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same product and bytes, with the split-K int32 partials in
 * a library-owned device array of PF_NOALLOC_SCRATCH_BYTES (64 MiB) per device,
 * held until the process ends, instead of a caller's workspace.  The array's
 * device address is looked up once per device (pf_init, or the first call on
 * that device); the call allocates nothing.  Every call on a device shares that
 * device's array, so calls that overlap in time on one device (different
 * streams, or host threads) race; the array keeps the last call's partials,
 * which every call overwrites before reading (nothing needs clearing).  Returns
 * PF_EWORKSPACE, before any device work, when the product's split plan needs
 * more than the array holds (pf_gemm_i8_chunk_workspace reports the need);
 * otherwise as pf_gemm_i8_chunk. */
#define PF_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
PF_API pf_status pf_gemm_i8_chunk_noalloc(const int8_t* W, const float* w_scale, int64_t N,
                                          int64_t K, const int8_t* xq, const float* a_scale,
                                          int64_t M, float* y, void* stream);

/* The per-token baseline ("Batched Prefill", §The Problem: one GEMV per token,
 * every weight re-read per token): y [N] = product of W with one token xq [K]. */
PF_API pf_status pf_gemv_i8(const int8_t* W, const float* w_scale, int64_t N, int64_t K,
                     const int8_t* xq, const float* a_scale, float* y, void* stream);

/* Projection set of one layer, in this order: q, k, v, o, gate, up, down.
 * Shapes: q, k, v, o [H][H]; gate, up [F][H]; down [H][F]; w_scale[j] has one
 * f32 per weight row. */
#define PF_NPROJ 7
typedef struct {
    const int8_t* W[PF_NPROJ];
    const float* w_scale[PF_NPROJ];
} pf_layer;

typedef struct {
    int64_t n_layers;
    int64_t hidden;          /* H */
    int64_t ffn;             /* F */
    const pf_layer* layers;  /* host array of n_layers */
    /* Optional (NULL: none): a second host array of n_layers describing a second
     * copy of the same weights at other addresses.  Chunk c reads its weights
     * from it when c is odd (the per-token mode ignores it); with equal contents
     * the results are unchanged.  Alternating two copies keeps one chunk's
     * weights from being served to the next by a last-level cache that can hold
     * one copy, so a caller can measure the rate of the weight stream from
     * DRAM alone. */
    const pf_layer* layers_alt;
    /* PF_ACT_NONE: down reads quantise(up).  PF_ACT_SWIGLU: down reads
     * quantise(r), r = fl(silu(gate) * up) elementwise with silu(g) =
     * fl(g / fl(1 + expf_cr(-g))) (expf_cr as pf_expf_cr), so gate feeds down
     * too.  The pages name gate, up and down projections but no activation;
     * the gated SiLU is the feed-forward of the model families they run.  With
     * no normalisation between layers the gated product is of degree two in
     * the layer input, so long chains of it grow or shrink without bound: it
     * suits stacks of a few layers (the expert layer is one). */
    int64_t activation;
    /* 0: no attention (o reads quantise(h), as q, k, v do).  n_heads > 0 adds
     * the causal attention of "Batched Prefill" (§What Stays Sequential: it
     * runs per position inside each chunk) over the K/V cache that the call
     * writes ("Single-pass prefill", "The fix": position t attends over the
     * K/V history kv_[layer][0..t]).  Per layer and token: q, k, v, gate, up
     * from quantise(h); k and v written to the cache; per head of d = H /
     * n_heads values, s_j = fl(dot(q, k_j) * c) over positions j = 0..t (the
     * dot an f32 sum in ascending index of separately rounded products,
     * c = fl(1 / fl(sqrt(d)))), m = max s_j, z_j = expf_cr(fl(s_j - m)),
     * S = the z_j summed in ascending j, p_j = fl(z_j / S), out = the
     * ascending-j sum of fl(p_j * v_j) from +0; then o = product of W_o with
     * quantise(out).  o feeds nothing further, so y is the same as without
     * attention.  Requires H % n_heads == 0, d % 4 == 0, d <= 256 and
     * H <= 8192. */
    int64_t n_heads;
} pf_stack;

#define PF_ACT_NONE 0
#define PF_ACT_SWIGLU 1

/* Statistics of one pf_prefill_stack call.  time_kernels and max_groups are
 * the inputs: set time_kernels to 1 to give every launch a pair of HIP events stamped when the kernel
 * itself starts and ends (hipExtLaunchKernelGGL) and get per-class device
 * times; kernels of the three chunk groups (one stream each) overlap in time,
 * so the summed launch durations (product_ms, quant_ms) can exceed the call's
 * elapsed time, while the busy times (the union of a class's launch intervals)
 * cannot.  Algorithmic bytes count what the method must move, once: for the
 * products of a (chunk, layer) pair the weights and their scales, one read of
 * the quantised tokens and their scales per phase (the six products that share
 * them read them once) and every f32 output written once; for a quantisation
 * the f32 inputs, the int8 codes and the scales.  Traffic that the schedule
 * adds (the down product's split-K int32 partials, written and read back) is
 * reported apart as overhead_bytes. */
typedef struct {
    int time_kernels;          /* in: 1 = time every launch                       */
    int max_groups;            /* in: at most this many chunk groups (0: the library's
                                  choice: 3 for chunks of up to 64 tokens, 2 above);
                                  1 runs every launch in order on the caller's
                                  stream, so no two launches overlap               */
    int groups;                /* out: chunk groups used                          */
    int per_token_mode;        /* out: 1 if the per-token GEMV path ran           */
    int64_t chunks;            /* chunks processed (the last may be ragged)       */
    int64_t tail_tokens;       /* tokens in the last chunk                        */
    int64_t launches;          /* kernel launches queued                          */
    double alg_bytes;          /* algorithmic bytes of all launches               */
    double elapsed_ms;         /* device time from before the first launch to after the last */
    int64_t product_launches;  /* int8 products (chunk GEMMs, or GEMVs per token) */
    int64_t quant_launches;    /* quantisations                                   */
    double product_alg_bytes;
    double quant_alg_bytes;
    double product_ms;         /* summed device time of the products (time_kernels) */
    double quant_ms;           /* summed device time of the quantisations (time_kernels) */
    double product_busy_ms;    /* time at least one product ran (time_kernels)    */
    double quant_busy_ms;      /* time at least one quantisation ran (time_kernels) */
    double overhead_bytes;     /* split-K partials written and read back          */
    int64_t attn_launches;     /* attention launches (stacks with n_heads > 0)    */
    double attn_alg_bytes;     /* q rows, the K/V history once per (chunk, layer), codes */
    double attn_ms;            /* summed device time of the attention launches    */
} pf_stack_stats;

/* Workspace bytes for pf_prefill_stack with this stack and chunk size. */
PF_API size_t pf_prefill_stack_workspace(const pf_stack* stack, int64_t chunk);

/* Sweeps a prompt of P tokens through every layer's projection set, one chunk
 * of `chunk` tokens at a time, the last chunk ragged ("Single-pass prefill",
 * "The fix"; "Batched Prefill", §The Solution).  Per chunk and layer, with h the
 * layer input (x for layer 0):
 *   (a, sa) = quantise(h); q, k, v, o, gate, up = products with a;
 *   (b, sb) = quantise(up); down = product with b; the next layer's h = down.
 * x [P][H] f32 -> y [P][H] f32 (the last layer's down).  proj, when not NULL,
 * receives every projection output: proj [L][P][5H + 2F] f32, each row holding
 * q, k, v, o, gate, up, down concatenated.  When NULL, the outputs nothing
 * reads are computed but not stored: q (unless the attention reads it), k and
 * v (the attention reads the cache), o, and gate without the gated SiLU; y
 * and kv are the same, with fewer bytes written.  kv, required when the stack has
 * n_heads > 0 (ignored otherwise), receives the K/V cache: kv [L][2][P][H] f32,
 * k of layer l and position t at kv[l][0][t], v at kv[l][1][t].  With the environment variable
 * PF_BATCHED_PREFILL=0 the same call runs one GEMV per token and projection
 * instead (the per-token baseline); the bytes of y and proj are identical
 * ("Batched Prefill", §Correctness).  stats, when not NULL, is filled in and the
 * call then synchronises the stream (see pf_stack_stats). */
PF_API pf_status pf_prefill_stack(const pf_stack* stack, const float* x, int64_t P, int64_t chunk,
                           float* y, float* proj, float* kv, void* workspace, size_t ws_bytes,
                           pf_stack_stats* stats, void* stream);

/* Statistics of one pf_prefill_stack_streamed call (filled when not NULL; the
 * call then synchronises the stream). */
typedef struct {
    int64_t n_buffers;         /* device ring slots                                */
    int64_t layers_copied;     /* host-to-device layer copies (one per layer)      */
    int64_t prefetch_hits;     /* copies complete before the previous layer's
                                  compute ended: the compute never waited          */
    int64_t prefetch_misses;   /* the others (the first layer's copy always)       */
    double bytes_copied;       /* weights and scales moved over the host link      */
    double elapsed_ms;         /* device time of the whole call                    */
} pf_stream_stats;

/* Workspace bytes for pf_prefill_stack_streamed: the device ring of n_buffers
 * layer slots and the activations of a P-token prompt. */
PF_API size_t pf_prefill_stack_streamed_workspace(const pf_stack* stack, int64_t P, int64_t n_buffers);

/* The stack with its weights in host memory, for models larger than device
 * memory ("Predictive prefetch", "The fix: an async double-buffer ring": while
 * layer L computes, layer L + 1 is materialised in the other buffer; a copy
 * that is ready when needed is a hit, one that is not is a miss and the
 * compute waits; "Single-pass prefill", "The fix": stream each layer once and
 * sweep every prompt position through it).  stack->layers hold HOST pointers
 * (pinned memory from hipHostMalloc, so the copies are asynchronous; read
 * during the call); layers_alt must be NULL and n_heads 0.  Layer l is copied
 * into ring slot l % n_buffers on a library-owned copy stream, at most
 * n_buffers - 1 layers ahead; the copy into a slot waits for the compute that
 * last used it; the compute of layer l runs every chunk of `chunk` tokens
 * through it and waits for its copy only before its first product.  The
 * results are those of pf_prefill_stack (the arithmetic is the same, only the
 * schedule differs; "Predictive prefetch", "Three backends, one truth"):
 * x [P][H] -> y [P][H].  n_buffers >= 2.  Calls that share a workspace must be
 * ordered. */
PF_API pf_status pf_prefill_stack_streamed(const pf_stack* stack, const float* x, int64_t P,
                                           int64_t chunk, float* y, int64_t n_buffers,
                                           void* workspace, size_t ws_bytes,
                                           pf_stream_stats* stats, void* stream);

/* Mixture-of-experts layer ("Red Lite dev24", What changed):
 *   W_router [E][H] f32; W_gate, W_up [E][I][H] int8; W_down [E][H][I] int8;
 *   s_gate, s_up [E][I] f32; s_down [E][H] f32. */
typedef struct {
    int64_t n_experts;   /* E */
    int64_t top_k;       /* experts per token */
    int64_t hidden;      /* H */
    int64_t inter;       /* I */
    const float* W_router;
    const int8_t* W_gate;
    const int8_t* W_up;
    const int8_t* W_down;
    const float* s_gate;
    const float* s_up;
    const float* s_down;
    int64_t activation;  /* PF_ACT_NONE: r = fl(g * u); PF_ACT_SWIGLU: r = fl(silu(g) * u) */
    int64_t renormalize; /* 0: weights = softmax p of the chosen experts; 1: divided by
                            their sum T (taken in rank order), w = fl(p / T)        */
} pf_moe;

/* Workspace bytes for pf_moe_chunk with T tokens. */
PF_API size_t pf_moe_chunk_workspace(const pf_moe* moe, int64_t T);

/* Expert prefill of one chunk of T tokens x [T][H] f32, all on the device:
 *   logits[t][e] = sum over k ascending of fl(W_router[e][k] * x[t][k]) (f32,
 *     each product and sum rounded on its own);
 *   p = softmax(logits[t]) with correctly rounded expf, normaliser summed in
 *     ascending e; ids[t] = the top_k experts by descending p, ties to the lower
 *     id; weights[t][j] = p[ids[t][j]] (not renormalised);
 *     (with renormalize, weights[t][j] = fl(p / T), T the chosen p summed in
 *     rank order);
 *   tokens are grouped by expert (the union of selected experts, tokens in
 *     ascending order within an expert) and each expert runs as int8 products
 *     over its group: g = gate(xq), u = up(xq), r = fl(g * u) (or
 *     fl(silu(g) * u) with PF_ACT_SWIGLU), (hq, hs) = quantise(r) per
 *     (token, expert) row, y_e = down(hq);
 *   out[t] = +0 then, over the selected experts in ascending id,
 *     out[t][j] = fl(out[t][j] + fl(weights_e * y_e[j])).
 * With the environment variable PF_MOE_FUSED=1 and hidden and inter each 512,
 * 1024 or 2048, gate/up, quantise(r) and down run as one launch with one
 * workgroup per expert ("Red Lite dev24", Scope boundary); the outputs are
 * identical.
 * ids [T][top_k] int32, weights [T][top_k] f32, out [T][H] f32.
 * Limits: T * top_k <= 65536, E <= 1024, top_k <= 32, T <= 16384. */
PF_API pf_status pf_moe_chunk(const pf_moe* moe, const float* x, int64_t T, int32_t* ids,
                       float* weights, float* out, void* workspace, size_t ws_bytes,
                       void* stream);

/* The correctly rounded binary32 exp used by the softmax above, applied
 * elementwise to x [n] -> y [n] (exposed so that it can be checked). */
PF_API pf_status pf_expf_cr(const float* x, int64_t n, float* y, void* stream);

#ifdef __cplusplus
}
#endif
#endif
