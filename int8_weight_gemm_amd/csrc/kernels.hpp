// kernels.hpp — kernel argument blocks and host-side launch wrappers of libprefill.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pf {

// Start/stop events for the next kernel launch of this host thread, or nulls.
// hipExtLaunchKernelGGL stamps them when the kernel itself starts and ends (the
// times a kernel-trace profiler reports), so a timed launch carries no
// dispatch latency in its measured duration.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
extern thread_local LaunchEvents t_launch_events;

#define PF_LAUNCH(KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                 \
    do {                                                                                  \
        if (::pf::t_launch_events.start)                                                  \
            hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM,                     \
                                  ::pf::t_launch_events.start, ::pf::t_launch_events.stop, \
                                  0, __VA_ARGS__);                                        \
        else                                                                              \
            hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);          \
    } while (0)

// One int8 product y[t][n] = epilogue(sum_k W[n][k] * X[t][k]) of a grouped launch.
struct GemmProb {
    const int8_t* W;      // [N][K]
    const float* ws;      // [N]
    const int8_t* X;      // [M][ldx]
    const float* xs;      // [M]
    float* Y;             // [M][ldy]
    float* Y2;            // optional second copy of the output [M][ldy2] (or null)
    int* acc;             // split-K int32 partials (or null): split s, token t, row n at
                          // acc[s * acc_split + t * acc_ld + n]
    int64_t acc_ld;       // ints between token rows of a split's partials
    int64_t acc_split;    // ints between splits
    int64_t ldx;          // bytes between token rows of X
    int64_t ldy;          // floats between token rows of Y
    int64_t ldy2;         // floats between token rows of Y2
    int N, K, M;
    int tiles_n;          // row tiles (16 rows skinny, 128 rows tiled)
    int tiles_m;          // token tiles (tiled kernel only)
    int splits;           // K splits across workgroups (skinny kernel only)
    int kb_per_split;     // 64-byte k-blocks per split
    int tile_begin;       // first flat workgroup index of this problem
};

constexpr int kMaxProbs = 8;
struct GemmSet {
    GemmProb p[kMaxProbs];
    int nprob;
    int total_tiles;
};

// One step of the chunk x layer sweep: up to kMaxPairs (chunk, layer) pairs,
// each multiplying its chunk's quantised tokens with the same projection slots
// (q..up, or down) of its own layer.  Workgroup b -> pair b / tiles_per_pair.
constexpr int kMaxPairs = 16;
constexpr int kComputeUnits = 256;          // MI355X (gfx950)
struct StepPair {
    const int8_t* W[6];
    const float* ws[6];
    const int8_t* X;      // quantised tokens [M][ldx]
    const float* xs;      // token scales [M]
    float* Y;             // output rows [M][ldy]; projection j at column yoff[j]
    float* Y2;            // optional second copy [M][ldy2] (single-projection steps) or null
    int* part;            // split-K int32 partials [splits][part_stride] (rows of ldp) or null
    float* kv[2];         // attention: the pair's K and V cache rows [M][ldkv] (projections
                          // kv_proj[0] and kv_proj[1] also store there) or null
    int M;
};
struct StackStep {
    StepPair pair[kMaxPairs];
    int npairs;
    int nproj;            // projections per pair (6 or 1)
    int K;
    int rows[6];          // rows of projection j
    int yoff[6];          // column of projection j inside an output row
    int tile_off[7];      // tile prefix over projections, per pair
    int tiles_m;          // token tiles (tiled kernel)
    int splits;           // K splits
    int partials;         // 1: store int32 partials to StepPair::part, no epilogue
    int kb_per_split;     // 64-byte k-blocks per split
    int64_t ldx, ldy, ldy2;
    int64_t ldp;          // int32 elements between token rows of the partials
    int64_t part_stride;  // int32 elements between splits of the partials
    int kv_proj[2];       // projections whose outputs also go to the K / V cache (-1: none)
    int64_t ldkv;         // floats between cache rows
    unsigned nostore;     // bit j: projection j's rows are not stored (nothing reads them);
                          // its cache rows still are
};

// The K or V cache row base of projection j of a pair (null: none).
__host__ __device__ inline float* step_kv(const StackStep& S, const StepPair& p, int j)
{
    return j == S.kv_proj[0] ? p.kv[0] : (j == S.kv_proj[1] ? p.kv[1] : nullptr);
}

// Causal attention of the tokens of up to kMaxPairs (chunk, layer) pairs, each
// token over cache positions 0 .. its own, followed by the per-token
// quantisation of the attention row.
struct AttnPair {
    const float* q;       // q rows of the pair's tokens [M][ldq]
    const float* K;       // the layer's K cache, position 0 [P][ldkv]
    const float* V;       // the layer's V cache, position 0
    int8_t* ao;           // quantised attention rows [M][H]
    float* sao;           // their scales [M]
    int pos0;             // position of the pair's first token
    int M;
};
struct AttnStep {
    AttnPair pair[kMaxPairs];
    int npairs;
    int max_m;            // tokens of the largest pair (workgroups per pair)
    int H, n_heads, d;
    float scale;          // fl(1 / fl(sqrt(d)))
    int64_t ldq, ldkv;
};
constexpr int kAttnMaxH = 8192;          // attention row held in LDS
constexpr int kAttnMaxD = 256;           // head width: four values per lane

// Per-token quantisation of several chunks' rows in one launch.  Mode 0: the
// rows are f32 [M][ld] at src.  Mode 1 (part != null): the rows are rebuilt
// first from split-K int32 partials of a product (sum over the splits, then the
// epilogue with the product's weight-row and token scales), written to h (and
// y when not null); q == null skips the quantisation itself.
constexpr int kMaxQuant = kMaxPairs + 1;
struct QuantPair {
    const float* src;     // mode 0 rows
    const float* gate;    // mode 0, optional: rows [M][ld] g; the row quantised is then
                          // r = fl(silu(g) * src), silu through the correctly rounded exp
    int8_t* q;            // [M][K] codes, or null
    float* s;             // [M] scales
    int64_t ld;           // floats between source rows
    int row0;             // first workgroup of this pair
    const int* part;      // mode 1: [splits][part_stride], rows of K int32
    int64_t part_stride;
    int splits;
    const float* ws;      // mode 1: weight-row scales [K]
    const float* as;      // mode 1: token scales [M]
    float* h;             // mode 1: rebuilt rows [M][ldh] (null: not stored; rows of at
                          // most 16384 values only)
    int64_t ldh;
    float* y;             // mode 1: optional copy [M][K]
};
struct QuantStep {
    QuantPair pair[kMaxQuant];
    int npairs;
    int K;
    int total_rows;
};

// Expert-grouped product: expert e multiplies its W_e with the rows of its token
// group (rows off[e] .. off[e+1] of the pair list).
struct ExpertArgs {
    const int8_t* W0;     // [E][N][K]
    const int8_t* W1;     // second weight with the same shape (gate/up pair) or null
    const float* s0;      // [E][N]
    const float* s1;      // [E][N] or null
    const int* off;       // [E+1] pair offsets per expert
    const int* gather;    // pair -> X row (token) or null: X row = pair index
    const int8_t* X;      // [rows][ldx]
    const float* xs;      // per X row
    float* Y;             // [pairs][ldy]
    int64_t ldx, ldy;
    int N, K, E;
    int tiles_n;
    int act;              // gate/up pair: 0 -> g * u; 1 -> silu(g) * u
};

// Host launch wrappers (return a hipError_t of the launch).
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_quantize(const float* x, int64_t ldx, int M, int K, int8_t* q, float* scale,
                           hipStream_t s);
hipError_t launch_quantize_step(const QuantStep& S, hipStream_t s);
// M rows r = fl(silu(gate) * up) (rows of both at stride ld) quantised per row.
hipError_t launch_quantize_gated(const float* up, const float* gate, int64_t ld, int M, int K,
                                 int8_t* q, float* scale, hipStream_t s);
hipError_t launch_gemv(const GemmSet& set, hipStream_t s);
hipError_t launch_gemm_tiled_step(const StackStep& S, int64_t M, hipStream_t s);
hipError_t launch_gemm_stream(const StackStep& S, int token_blocks, hipStream_t s);
// K-blocks per split the token-resident product takes: 16 up to 64 tokens, 8 for
// 65 to 128 tokens (run as eight 16-token blocks).
constexpr int xres_max_kb(int token_blocks) { return token_blocks <= 4 ? 16 : 8; }
hipError_t launch_gemm_xres(const StackStep& S, int token_blocks, hipStream_t s);
hipError_t launch_gemm_skinny(const GemmSet& set, int token_blocks, hipStream_t s);
hipError_t launch_gemm_tiled(const GemmSet& set, int tile_tokens, hipStream_t s);
hipError_t launch_split_reduce(const GemmSet& set, hipStream_t s);
// Tiled product tiles: 256 weight rows x 256 or 128 tokens; tiled_tokens(M) is
// the stack sweep's choice (pf_gemm_i8_chunk plans its own).
constexpr int kTiledRows = 256;
int tiled_tokens(int64_t M);

// Router logits; with xq non-null the same launch quantises x per token into
// xq [T][H] and xs [T].
hipError_t launch_router(const float* Wr, const float* x, int E, int H, int T, float* logits,
                         int8_t* xq, float* xs, hipStream_t s);
hipError_t launch_softmax_topk(const float* logits, int E, int T, int k, int renorm, int* ids,
                               float* w, hipStream_t s);
hipError_t launch_group(const int* ids, const float* w, int T, int k, int E, int* off,
                        int* pair_tok, int* comb_row, float* comb_w, hipStream_t s);
hipError_t launch_expert(const ExpertArgs& a, hipStream_t s);
// gate/up, the per-row quantisation of r and down of every expert in one
// launch (one workgroup per expert); G.Y receives r, Dn.Y the pairs' outputs.
// For hidden and inter sizes of 512, 1024 or 2048 (expert_fused_shape).
bool expert_fused_shape(int64_t H, int64_t I);
hipError_t launch_expert_fused(const ExpertArgs& G, const ExpertArgs& Dn, hipStream_t s);
hipError_t launch_combine(const float* ypair, const int* comb_row, const float* comb_w, int T,
                          int k, int H, float* out, hipStream_t s);
hipError_t launch_expf(const float* x, int64_t n, float* y, hipStream_t s);
hipError_t launch_attention(const AttnStep& S, hipStream_t s);

// Sizes of the grouping kernel's shared bitmap.
inline size_t group_lds_bytes(int T, int E) { return (size_t)E * ((T + 31) / 32) * 4; }

}  // namespace pf
