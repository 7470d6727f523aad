// api.hip — the C ABI of libprefill (include/libprefill.h): argument checks,
// workspace carving, kernel choice and launch order.  No device memory is
// allocated here; every call queues work on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <mutex>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/libprefill.h"
#include "kernels.hpp"

using namespace pf;

thread_local pf::LaunchEvents pf::t_launch_events;

namespace {

constexpr int64_t kMaxK = 131072;
constexpr size_t kAlign = 256;

// Per-device result of the architecture check: 0 unknown, 1 gfx950, -1 other.
std::atomic<int> g_arch[64];

pf_status check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return PF_ENODEV;
    }
    int v = g_arch[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return PF_ENODEV;
        }
        v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_arch[dev].store(v, std::memory_order_relaxed);
    }
    return v == 1 ? PF_OK : PF_ENODEV;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool valid_k(int64_t K) { return K > 0 && K % 64 == 0 && K <= kMaxK; }

pf_status launched(hipError_t e)
{
    if (e == hipSuccess) return PF_OK;
    (void)hipGetLastError();
    return PF_ELAUNCH;
}

// ---------------------------------------------------------------------------
// Split plan of the skinny product: 64-row tiles; when a launch has fewer tiles
// than compute units, the K range is split across workgroups (each split at
// least 8 k-blocks of 64 bytes) until every compute unit has one.
struct SkinnyPlan {
    int tiles_n, splits, kb_per_split;
    int tokens = 0;       // tiled products: tokens per tile (128 or 256)
};

constexpr int kSkinnyRows = 64;

SkinnyPlan plan_skinny(int64_t N, int64_t K, int64_t total_tiles)
{
    SkinnyPlan p;
    p.tiles_n = (int)((N + kSkinnyRows - 1) / kSkinnyRows);
    const int nkb = (int)(K / 64);
    int s = 1;
    while (total_tiles * s < kComputeUnits && nkb / (2 * s) >= 8) s *= 2;
    p.kb_per_split = (nkb + s - 1) / s;
    p.splits = (nkb + p.kb_per_split - 1) / p.kb_per_split;
    return p;
}

SkinnyPlan unsplit(int64_t N, int64_t K)
{
    return SkinnyPlan{(int)((N + kSkinnyRows - 1) / kSkinnyRows), 1, (int)(K / 64), 0};
}

// Plan of a standalone product of at most 64 tokens; xres_shape: the output
// rows suit the token-resident kernel (16-byte aligned, N a multiple of 4).
SkinnyPlan plan_chunk_small(int64_t N, int64_t K, bool xres_shape)
{
    SkinnyPlan p = plan_skinny(N, K, (N + kSkinnyRows - 1) / kSkinnyRows);
    // splits longer than the token-resident kernel takes: with enough tiles
    // for half the compute units the streamed kernel runs the whole K per
    // tile (no partials, no second launch)
    if (p.kb_per_split > 16 && p.tiles_n >= kComputeUnits / 2) p = unsplit(N, K);
    // a product of at most a few MB is over before a second launch (the
    // split's reduction) would start: split only as far as the token-resident
    // kernel needs (16 k-blocks per split)
    if (N * K <= (8 << 20) && xres_shape) {
        const int nkb = (int)(K / 64);
        const int sp = (nkb + 15) / 16;
        p.kb_per_split = (nkb + sp - 1) / sp;
        p.splits = (nkb + p.kb_per_split - 1) / p.kb_per_split;
    }
    return p;
}

size_t split_bytes(int64_t N, int64_t M, const SkinnyPlan& p)
{
    if (p.splits <= 1) return 0;
    return round_up((size_t)p.splits * (size_t)M * (size_t)N * 4, kAlign);
}

int token_blocks(int64_t M) { return (int)((M + 15) / 16); }

// Fills a skinny problem.  With a split plan its int32 accumulator ([m_alloc][N],
// m_alloc >= M) and counters are carved from `scratch`, which then advances.
void make_skinny(GemmProb& g, const int8_t* W, const float* ws, int64_t N, int64_t K,
                 const int8_t* X, int64_t ldx, const float* xs, int64_t M, float* Y, int64_t ldy,
                 const SkinnyPlan& p, char*& scratch, int64_t m_alloc)
{
    std::memset(&g, 0, sizeof(g));
    g.W = W; g.ws = ws; g.X = X; g.xs = xs; g.Y = Y;
    g.ldx = ldx; g.ldy = ldy;
    g.N = (int)N; g.K = (int)K; g.M = (int)M;
    g.tiles_n = p.tiles_n; g.tiles_m = 1;
    g.splits = p.splits; g.kb_per_split = p.kb_per_split;
    if (p.splits > 1) {
        g.acc = reinterpret_cast<int*>(scratch);
        g.acc_ld = N;
        g.acc_split = M * N;
        scratch += split_bytes(N, m_alloc, p);
    }
}

// Tiled product plan: tiles of 256 weight rows x 256 or 128 tokens, and the K
// range possibly split across workgroups (each split at least 8 k-blocks), the
// splits' int32 partials summed by k_split_reduce.  Tile width and split count
// minimise a cost estimate: rounds of work units over the compute units x
// (k-blocks per split + the ~6 stages a unit spends filling and draining its
// pipeline) x the stage time of the width (~1.2 us at 256 tokens, ~0.85 us at
// 128), plus the partials' write and read at ~4 TB/s and one more launch.
// The estimate follows measured times within a few per cent on products of
// 4096-38400 rows and 128-512 tokens.  max_splits = 1 plans without a split.
SkinnyPlan plan_tiled(int64_t N, int64_t K, int64_t M, int max_splits = 16)
{
    SkinnyPlan best{};
    double best_us = 0.0;
    const int nkb = (int)(K / 64);
    const int tiles_n = (int)((N + kTiledRows - 1) / kTiledRows);
    for (int tw = 256; tw >= 128; tw /= 2) {
        if (tw == 256 && M <= 128) continue;
        const int64_t tiles = tiles_n * ((M + tw - 1) / tw);
        const double stage_us = tw == 256 ? 1.2 : 0.85;
        for (int sp = 1; sp <= max_splits && (sp == 1 || nkb / sp >= 8); sp *= 2) {
            int kbs = (nkb + sp - 1) / sp;
            if (kbs > 1 && (kbs & 1)) ++kbs;   // even: a split starts on a 128-byte line
            const int splits = (nkb + kbs - 1) / kbs;
            const int64_t rounds = (tiles * splits + kComputeUnits - 1) / kComputeUnits;
            double us = (double)rounds * (kbs + 6) * stage_us;
            if (splits > 1) us += 2.0 * splits * (double)M * (double)N * 4 / 4.0e6 + 3.0;
            if (best.tokens == 0 || us < best_us) {
                best = SkinnyPlan{tiles_n, splits, kbs, tw};
                best_us = us;
            }
        }
    }
    return best;
}

// Fills a tiled problem; with a split plan its partials ([splits][M][N]) are
// carved from `scratch`, which then advances.
void make_tiled(GemmProb& g, const int8_t* W, const float* ws, int64_t N, int64_t K,
                const int8_t* X, int64_t ldx, const float* xs, int64_t M, float* Y, int64_t ldy,
                const SkinnyPlan& p, char*& scratch)
{
    std::memset(&g, 0, sizeof(g));
    g.W = W; g.ws = ws; g.X = X; g.xs = xs; g.Y = Y;
    g.ldx = ldx; g.ldy = ldy;
    g.N = (int)N; g.K = (int)K; g.M = (int)M;
    g.tiles_n = p.tiles_n;
    g.tiles_m = (int)((M + p.tokens - 1) / p.tokens);
    g.splits = p.splits; g.kb_per_split = p.kb_per_split;
    if (p.splits > 1) {
        g.acc = reinterpret_cast<int*>(scratch);
        g.acc_ld = N;
        g.acc_split = M * N;
        scratch += split_bytes(N, M, p);
    }
}

void finish_set(GemmSet& set, int kind)  // kind 0 gemv, 1 skinny, 2 tiled
{
    int begin = 0;
    for (int i = 0; i < set.nprob; ++i) {
        GemmProb& g = set.p[i];
        g.tile_begin = begin;
        if (kind == 0) begin += (g.N + 15) / 16;
        else if (kind == 1) begin += g.tiles_n * g.splits;
        else begin += g.tiles_n * g.tiles_m * g.splits;
    }
    set.total_tiles = begin;
}

// One skinny problem through the token-resident kernel: the same work items
// (64-row tiles x K splits of at most 16 k-blocks); with a split its int32
// partials go to the problem's accumulator and k_split_reduce applies the
// epilogue.  Needs 16-byte aligned output rows (four-row stores).
bool xres_fits_shape(int64_t N, const float* y)
{
    return (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
}

bool xres_fits(const GemmProb& g)
{
    return g.kb_per_split <= 16 && (g.N & 3) == 0 && ((reinterpret_cast<uintptr_t>(g.Y) & 15) == 0) &&
           (g.ldy & 3) == 0 && !g.Y2;
}

pf_status run_skinny_xres(GemmSet& set, int64_t M, hipStream_t s)
{
    const GemmProb& g = set.p[0];
    StackStep S;
    std::memset(&S, 0, sizeof(S));
    S.npairs = 1;
    S.nproj = 1;
    S.K = g.K;
    S.rows[0] = g.N;
    S.tile_off[1] = (g.N + kSkinnyRows - 1) / kSkinnyRows;
    S.tiles_m = 1;
    S.splits = g.splits;
    S.partials = g.splits > 1 ? 1 : 0;
    S.kb_per_split = g.kb_per_split;
    S.ldx = g.ldx;
    S.ldy = g.ldy;
    S.ldp = g.acc_ld;
    S.part_stride = g.acc_split;
    StepPair& p = S.pair[0];
    p.W[0] = g.W;
    p.ws[0] = g.ws;
    p.X = g.X;
    p.xs = g.xs;
    p.Y = g.Y;
    p.part = g.acc;
    p.M = g.M;
    if (pf_status st = launched(launch_gemm_xres(S, token_blocks(M), s))) return st;
    if (g.splits <= 1) return PF_OK;
    finish_set(set, 1);
    return launched(launch_split_reduce(set, s));
}

// Runs a set of products that share M (skinny for M <= 64, tiled above, with
// tiles of `tile_tokens` tokens).
// One unsplit skinny problem through the streamed step kernel (weights and
// token pieces copied per stage, any K, any output alignment).
pf_status run_skinny_stream(GemmSet& set, int64_t M, hipStream_t s)
{
    const GemmProb& g = set.p[0];
    StackStep S;
    std::memset(&S, 0, sizeof(S));
    S.npairs = 1;
    S.nproj = 1;
    S.K = g.K;
    S.rows[0] = g.N;
    S.tile_off[1] = (g.N + kSkinnyRows - 1) / kSkinnyRows;
    S.tiles_m = 1;
    S.splits = 1;
    S.kb_per_split = g.K / 64;
    S.ldx = g.ldx;
    S.ldy = g.ldy;
    StepPair& p = S.pair[0];
    p.W[0] = g.W;
    p.ws[0] = g.ws;
    p.X = g.X;
    p.xs = g.xs;
    p.Y = g.Y;
    p.M = g.M;
    return launched(launch_gemm_stream(S, token_blocks(M), s));
}

pf_status run_products(GemmSet& set, int64_t M, int tile_tokens, hipStream_t s)
{
    if (M <= 64) {
        if (set.nprob == 1 && xres_fits(set.p[0])) return run_skinny_xres(set, M, s);
        if (set.nprob == 1 && set.p[0].splits == 1) return run_skinny_stream(set, M, s);
        finish_set(set, 1);
        return launched(launch_gemm_skinny(set, token_blocks(M), s));
    }
    finish_set(set, 2);
    return launched(launch_gemm_tiled(set, tile_tokens, s));
}

// ---------------------------------------------------------------------------
// Stack workspace: `slots` chunk slots, each with the quantised layer input
// a [chunk][H], the quantised up output b [chunk][F], their scales, and the
// projection rows [chunk][5H+2F] used when the caller keeps none.  A chunk in
// flight owns one slot for all of its layers.
struct StackLayout {
    int groups;           // chunk groups (one stream each)
    int gslots;           // slots per group: chunks of a group in flight at once
    int slots;
    int dsplits;          // K splits of the down product
    int dkb;              // k-blocks per down-product split
    size_t a, b, sa, sb, proj, part, ao, sao, slot_bytes, total;
};


constexpr int kMaxGroups = 4;

// Chunk groups of the stack sweep and the slots of each: three groups (the
// caller's stream and two library streams, within the four hardware queues a
// process gets by default) of up to 16 chunks in flight.  A step of a group
// launches one product over all of its chunks in flight, so a group's slots
// are at most kMaxPairs.
constexpr int kStackGroups = 3;
constexpr int kGroupSlots = 16;
constexpr int kGroupSlotsTiled = 4;  // chunks over 64 tokens: each product fills the chip
constexpr int kTiledGroups = 2;      // chunk groups over 64 tokens
static_assert(kStackGroups <= kMaxGroups && kGroupSlots <= kMaxPairs, "stack sweep shape");
static_assert(kTiledGroups <= kStackGroups, "a stream per group");

StackLayout stack_layout(int64_t L, int64_t H, int64_t F, int64_t chunk, bool attn)
{
    StackLayout S{};
    // chunks over 64 tokens: two groups, whose launches each carry up to two of
    // the 7B-class prompt's four 512-token chunks.  Every tile of a launch ends
    // at about the same time and then stores its 256 KB of outputs, so in one
    // group all compute units wait on the same burst of stores; two groups on
    // two streams run their launches out of phase (the prompt in 15.65 ms
    // against 16.25 ms in one group and 16.36 ms in three, on one box).
    S.groups = chunk <= 64 ? kStackGroups : kTiledGroups;
    S.gslots = (int)std::min<int64_t>(L, chunk <= 64 ? kGroupSlots : kGroupSlotsTiled);
    S.slots = S.groups * S.gslots;
    // down-product K splits: on the skinny path at most 16 k-blocks (the
    // token slice in LDS) each.  On the tiled path two, when a group's down
    // launch (gslots chunks of 256-row x tile-width tiles) would leave compute
    // units idle: the 7B-class stack at 512 tokens in two groups ran its
    // prompt in 15.65 ms split in two against 16.26 ms unsplit and 16.64 ms
    // in four.
    const int nkb = (int)(F / 64);
    const int64_t down_tiles = S.gslots * ((H + kTiledRows - 1) / kTiledRows) *
                               ((chunk + tiled_tokens(chunk) - 1) / tiled_tokens(chunk));
    const int want = chunk <= 64 ? (nkb + 15) / 16 : (down_tiles < kComputeUnits && nkb >= 16 ? 2 : 1);
    S.dkb = (nkb + want - 1) / want;
    S.dsplits = (nkb + S.dkb - 1) / S.dkb;
    size_t o = 0;
    S.a = o; o += round_up((size_t)chunk * H, kAlign);
    S.b = o; o += round_up((size_t)chunk * F, kAlign);
    S.sa = o; o += round_up((size_t)chunk * 4, kAlign);
    S.sb = o; o += round_up((size_t)chunk * 4, kAlign);
    S.proj = o; o += round_up((size_t)chunk * (5 * H + 2 * F) * 4, kAlign);
    S.part = o; o += (chunk <= 64 || S.dsplits > 1) ? round_up((size_t)S.dsplits * chunk * H * 4, kAlign) : 0;
    // attention: the quantised attention rows of the chunk and their scales
    S.ao = o; o += attn ? round_up((size_t)chunk * H, kAlign) : 0;
    S.sao = o; o += attn ? round_up((size_t)chunk * 4, kAlign) : 0;
    S.slot_bytes = o;
    S.total = o * S.slots;
    return S;
}

pf_status validate_stack(const pf_stack* st)
{
    if (!st || !st->layers || st->n_layers <= 0 || st->hidden <= 0 || st->ffn <= 0)
        return PF_EINVAL;
    if (st->activation != PF_ACT_NONE && st->activation != PF_ACT_SWIGLU) return PF_EINVAL;
    if (st->n_heads < 0) return PF_EINVAL;
    if (st->n_heads > 0) {
        const int64_t d = st->hidden / st->n_heads;
        if (st->hidden % st->n_heads != 0 || d % 4 != 0 || d > kAttnMaxD || st->hidden > kAttnMaxH)
            return PF_EINVAL;
    }
    if (!valid_k(st->hidden) || !valid_k(st->ffn)) return PF_EINVAL;
    if ((uint64_t)st->hidden * (uint64_t)st->ffn >= (1ull << 32)) return PF_EINVAL;   // 32-bit offsets
    for (const pf_layer* tab : {st->layers, st->layers_alt}) {
        if (!tab) continue;
        for (int64_t l = 0; l < st->n_layers; ++l)
            for (int j = 0; j < PF_NPROJ; ++j) {
                const pf_layer& ly = tab[l];
                if (!ly.W[j] || !ly.w_scale[j] || !aligned16(ly.W[j]) || !aligned4(ly.w_scale[j]))
                    return PF_EINVAL;
            }
    }
    return PF_OK;
}

bool per_token_mode()
{
    const char* v = std::getenv("PF_BATCHED_PREFILL");
    return v && v[0] == '0' && v[1] == '\0';
}

// PF_MOE_FUSED=1: the experts of pf_moe_chunk as one fused launch (measured a
// little slower than the three launches it replaces, so not the default).
bool moe_fused_mode()
{
    const char* v = std::getenv("PF_MOE_FUSED");
    return v && v[0] == '1' && v[1] == '\0';
}

// ---------------------------------------------------------------------------
// MoE workspace layout.
struct MoeLayout {
    size_t xq, xs, logits, off, pair_tok, comb_row, comb_w, r, hq, hs, ypair, total;
};

MoeLayout moe_layout(const pf_moe* m, int64_t T)
{
    MoeLayout L{};
    const size_t P = (size_t)T * m->top_k;
    size_t o = 0;
    L.xq = o; o += round_up((size_t)T * m->hidden, kAlign);
    L.xs = o; o += round_up((size_t)T * 4, kAlign);
    L.logits = o; o += round_up((size_t)T * m->n_experts * 4, kAlign);
    L.off = o; o += round_up((size_t)(m->n_experts + 1) * 4, kAlign);
    L.pair_tok = o; o += round_up(P * 4, kAlign);
    L.comb_row = o; o += round_up(P * 4, kAlign);
    L.comb_w = o; o += round_up(P * 4, kAlign);
    L.r = o; o += round_up(P * m->inter * 4, kAlign);
    L.hq = o; o += round_up(P * m->inter, kAlign);
    L.hs = o; o += round_up(P * 4, kAlign);
    L.ypair = o; o += round_up(P * m->hidden * 4, kAlign);
    L.total = o;
    return L;
}

pf_status validate_moe(const pf_moe* m)
{
    if (!m) return PF_EINVAL;
    if (m->n_experts <= 0 || m->n_experts > 1024 || m->top_k <= 0 || m->top_k > 32 ||
        m->top_k > m->n_experts)
        return PF_EINVAL;
    if (!valid_k(m->hidden) || !valid_k(m->inter)) return PF_EINVAL;
    if ((m->activation != PF_ACT_NONE && m->activation != PF_ACT_SWIGLU) ||
        (m->renormalize != 0 && m->renormalize != 1))
        return PF_EINVAL;
    const void* mats[] = {m->W_router, m->W_gate, m->W_up, m->W_down};
    for (const void* p : mats)
        if (!p || !aligned16(p)) return PF_EINVAL;
    const void* scales[] = {m->s_gate, m->s_up, m->s_down};
    for (const void* p : scales)
        if (!p || !aligned4(p)) return PF_EINVAL;
    return PF_OK;
}


// Algorithmic bytes of one product: weights, their scales, the quantised tokens
// and their scales read once, the f32 outputs written once.
double product_bytes(int64_t N, int64_t K, int64_t M)
{
    return (double)N * K + 4.0 * N + (double)M * K + 4.0 * M + 4.0 * M * N;
}

// The same without the token read, for products that share one token read.
double weight_out_bytes(int64_t N, int64_t K, int64_t M)
{
    return (double)N * K + 4.0 * N + 4.0 * M * N;
}

// Library-owned streams per device, one per chunk group after the first, which
// runs on the caller's stream (default priority, non-blocking), and the events
// that fork them from and join them back to the caller's stream.
// Created on first use and kept until the process ends; the mutex serialises
// calls that use them from several host threads.
struct DevStreams {
    std::mutex mu;
    bool ready = false;
    hipStream_t s[kMaxGroups] = {};
    hipEvent_t fork = nullptr;
    hipEvent_t join[kMaxGroups] = {};
    hipEvent_t kvdone[kMaxGroups][2] = {};   // a group's K/V cache rows of a step, by step parity
    hipStream_t copy = nullptr;              // host-to-device weight copies (streamed stacks)
};
DevStreams g_streams[64];

DevStreams* dev_streams()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    DevStreams* d = &g_streams[dev];
    return d;
}

pf_status ensure_streams(DevStreams* d)
{
    if (d->ready) return PF_OK;
    for (int i = 1; i < kStackGroups; ++i)
        if (hipStreamCreateWithFlags(&d->s[i], hipStreamNonBlocking) != hipSuccess) return PF_ELAUNCH;
    if (hipEventCreateWithFlags(&d->fork, hipEventDisableTiming) != hipSuccess) return PF_ELAUNCH;
    for (int i = 1; i < kStackGroups; ++i)
        if (hipEventCreateWithFlags(&d->join[i], hipEventDisableTiming) != hipSuccess) return PF_ELAUNCH;
    for (int i = 0; i < kStackGroups; ++i)
        for (int p = 0; p < 2; ++p)
            if (hipEventCreateWithFlags(&d->kvdone[i][p], hipEventDisableTiming) != hipSuccess)
                return PF_ELAUNCH;
    d->ready = true;
    return PF_OK;
}

// Launch bookkeeping of pf_prefill_stack: counts launches and algorithmic
// bytes per kernel class and, when asked, brackets every launch with a pair of
// HIP events on the caller's stream to time it.
class Recorder {
public:
    enum Kind { kQuant = 0, kProduct = 1, kAttn = 2, kKinds = 3 };
    Recorder(hipStream_t s, bool on, bool timed) : s_(s), on_(on), timed_(timed) {}
    ~Recorder()
    {
        for (auto& e : events_) (void)hipEventDestroy(e);
        if (t0_) (void)hipEventDestroy(t0_);
        if (t1_) (void)hipEventDestroy(t1_);
    }
    pf_status begin()
    {
        if (!on_) return PF_OK;
        if (hipEventCreate(&t0_) != hipSuccess || hipEventCreate(&t1_) != hipSuccess ||
            hipEventRecord(t0_, s_) != hipSuccess)
            return fail();
        return PF_OK;
    }
    template <class F>
    pf_status run(Kind k, double bytes, F&& launch, hipStream_t on = nullptr)
    {
        (void)on;
        hipEvent_t e0 = nullptr, e1 = nullptr;
        if (timed_) {
            if (hipEventCreate(&e0) != hipSuccess) return fail();
            events_.push_back(e0);
            if (hipEventCreate(&e1) != hipSuccess) return fail();
            events_.push_back(e1);
            t_launch_events = LaunchEvents{e0, e1};   // stamped at kernel start and end
        }
        const pf_status st = launch();
        t_launch_events = LaunchEvents{};
        if (st) return st;
        ++launches_[k];
        bytes_[k] += bytes;
        if (timed_) kinds_.push_back(k);
        return PF_OK;
    }
    void overhead(double bytes) { overhead_ += bytes; }
    pf_status end()
    {
        if (!on_) return PF_OK;
        if (hipEventRecord(t1_, s_) != hipSuccess || hipEventSynchronize(t1_) != hipSuccess)
            return fail();
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, t0_, t1_) != hipSuccess) return fail();
        total_ms_ = ms;
        // per launch its own duration, and its interval on the call's clock
        // (launches of different chunk groups may overlap in time)
        std::vector<std::pair<double, double>> iv[kKinds];
        for (size_t i = 0; i < kinds_.size(); ++i) {
            float a = 0.0f, b = 0.0f;
            if (hipEventElapsedTime(&ms, events_[2 * i], events_[2 * i + 1]) != hipSuccess ||
                hipEventElapsedTime(&a, t0_, events_[2 * i]) != hipSuccess ||
                hipEventElapsedTime(&b, t0_, events_[2 * i + 1]) != hipSuccess)
                return fail();
            ms_[kinds_[i]] += ms;
            iv[kinds_[i]].emplace_back(a, b);
        }
        // busy time of a kernel class: the union of its launches' intervals
        for (int k = 0; k < kKinds; ++k) {
            std::sort(iv[k].begin(), iv[k].end());
            double busy = 0.0, lo = 0.0, hi = -1.0;
            for (const auto& p : iv[k]) {
                if (p.first > hi) {
                    if (hi > lo) busy += hi - lo;
                    lo = p.first;
                    hi = p.second;
                } else {
                    hi = std::max(hi, p.second);
                }
            }
            if (hi > lo) busy += hi - lo;
            busy_[k] = busy;
        }
        return PF_OK;
    }
    void fill(pf_stack_stats* st) const
    {
        st->launches = launches_[0] + launches_[1] + launches_[2];
        st->alg_bytes = bytes_[0] + bytes_[1] + bytes_[2];
        st->elapsed_ms = total_ms_;
        st->quant_launches = launches_[kQuant];
        st->product_launches = launches_[kProduct];
        st->quant_alg_bytes = bytes_[kQuant];
        st->product_alg_bytes = bytes_[kProduct];
        st->quant_ms = timed_ ? ms_[kQuant] : 0.0;
        st->product_ms = timed_ ? ms_[kProduct] : 0.0;
        st->quant_busy_ms = timed_ ? busy_[kQuant] : 0.0;
        st->product_busy_ms = timed_ ? busy_[kProduct] : 0.0;
        st->overhead_bytes = overhead_;
        st->attn_launches = launches_[kAttn];
        st->attn_alg_bytes = bytes_[kAttn];
        st->attn_ms = timed_ ? ms_[kAttn] : 0.0;
    }

private:
    pf_status fail()
    {
        (void)hipGetLastError();
        return PF_ELAUNCH;
    }
    hipStream_t s_;
    bool on_, timed_;
    hipEvent_t t0_ = nullptr, t1_ = nullptr;
    std::vector<hipEvent_t> events_;
    std::vector<int> kinds_;
    int64_t launches_[kKinds] = {0, 0, 0};
    double bytes_[kKinds] = {0.0, 0.0, 0.0};
    double ms_[kKinds] = {0.0, 0.0, 0.0};
    double busy_[kKinds] = {0.0, 0.0, 0.0};
    double overhead_ = 0.0;
    double total_ms_ = 0.0;
};


// One pf_prefill_stack call.  Two schedules give the same bytes:
//   sweep():     chunk c reaches layer l at step start(c) + l, so one step runs
//                the (chunk, layer) pairs of a diagonal together: each pair
//                still reads its own layer's weights once for its chunk, and a
//                launch streams up to 16 layers' weights at once.  At most
//                `slots` chunks are in flight; chunk c waits for chunk c - slots.
//                Per step: quantise the layer inputs, the six K = H products,
//                quantise up, the down product.
//   per_token(): one token at a time, one GEMV per projection (the baseline).
struct StackRun {
    const pf_stack* st;
    const float* x;
    int64_t P, ch;
    float* y;
    float* proj;
    float* kv;             // K/V cache [L][2][P][H] (attention), or null
    char* ws;
    StackLayout lay;
    hipStream_t s;
    int ng = 1;            // chunk groups, each on its own stream (chunk c in group c % ng)
    DevStreams* ds = nullptr;
    hipStream_t gs[kMaxGroups] = {};

    bool attn() const { return st->n_heads > 0; }
    // the cache rows of (layer l, position p0): K at half 0, V at half 1
    float* kv_rows(int64_t l, int half, int64_t p0) const
    {
        return kv + (((size_t)l * 2 + half) * P + p0) * H();
    }

    // the layer table chunk c reads (the second copy for odd chunks, if any)
    const pf_layer& layer(int64_t c, int64_t l) const
    {
        return (st->layers_alt && (c & 1)) ? st->layers_alt[l] : st->layers[l];
    }
    int64_t H() const { return st->hidden; }
    int64_t F() const { return st->ffn; }
    int64_t NT() const { return 5 * st->hidden + 2 * st->ffn; }
    int64_t L() const { return st->n_layers; }
    int64_t gslots() const { return lay.gslots; }
    // a chunk in flight owns one slot of its group for all of its layers
    char* slot(int64_t c) const
    {
        const int64_t g = c % ng, k = c / ng;
        return ws + (size_t)(g * gslots() + k % gslots()) * lay.slot_bytes;
    }
    // projection rows of (chunk c, layer l): [M][NT], q..down concatenated
    float* rows(int64_t c, int64_t l) const
    {
        if (proj) return proj + ((size_t)l * P + (size_t)c * ch) * NT();
        return reinterpret_cast<float*>(slot(c) + lay.proj);
    }
    // Launch slots whose projection rows nothing reads when the caller keeps
    // none: q (unless the attention reads it), k and v (the attention reads
    // the cache), o, and gate without the gated SiLU; up feeds the down
    // product.  Those rows are not stored (the same bits come out in y and
    // the cache, with fewer bytes written).
    unsigned unread_rows(const int* projs, int n) const
    {
        if (proj) return 0u;
        unsigned m = 0;
        for (int j = 0; j < n; ++j) {
            const int p = projs[j];
            const bool read = p == 5 || (p == 4 && st->activation == PF_ACT_SWIGLU) || (p == 0 && attn());
            if (!read) m |= 1u << j;
        }
        return m;
    }
    int64_t offs(int j) const
    {
        const int64_t o[PF_NPROJ] = {0, H(), 2 * H(), 3 * H(), 4 * H(), 4 * H() + F(), 4 * H() + 2 * F()};
        return o[j];
    }
    // step at which the group's k-th chunk enters layer 0: one step after the
    // previous chunk, and never before the chunk gslots() earlier has left
    int64_t start(int64_t k) const
    {
        const int64_t S = gslots();
        return k + (k / S) * std::max<int64_t>(L() - S, 0);
    }
    int64_t chunks() const { return (P + ch - 1) / ch; }
    int64_t group_chunks(int g) const { return (chunks() - g + ng - 1) / ng; }
    int64_t group_steps(int g) const
    {
        const int64_t K = group_chunks(g);
        return K > 0 ? start(K - 1) + L() : 0;
    }

    // Chunks run in `ng` independent groups, one stream each, so that one
    // group's launches fill the start-up and tail of the other's.
    pf_status sweep(Recorder& rec)
    {
        gs[0] = s;
        if (ng == 1) {
            int64_t fin = -1;
            for (int64_t step = 0; step <= group_steps(0); ++step)
                if (pf_status r = group_step(rec, 0, step, fin, s)) return r;
            return PF_OK;
        }
        // group 0 runs on the caller's stream, the others on library streams
        for (int g = 1; g < ng; ++g) gs[g] = ds->s[g];
        if (hipEventRecord(ds->fork, s) != hipSuccess) return PF_ELAUNCH;
        for (int g = 1; g < ng; ++g)
            if (hipStreamWaitEvent(gs[g], ds->fork, 0) != hipSuccess) return PF_ELAUNCH;
        int64_t fin[kMaxGroups] = {-1, -1, -1, -1};
        int64_t nst = 0;
        for (int g = 0; g < ng; ++g) nst = std::max(nst, group_steps(g));
        for (int64_t step = 0; step <= nst; ++step)
            for (int g = 0; g < ng; ++g) {
                if (step <= group_steps(g)) {
                    if (pf_status r = group_step(rec, g, step, fin[g], gs[g])) return r;
                } else if (attn()) {
                    // a finished group keeps its step marks current (they cover all its work)
                    if (hipEventRecord(ds->kvdone[g][step & 1], gs[g]) != hipSuccess) return PF_ELAUNCH;
                }
            }
        for (int g = 1; g < ng; ++g) {
            if (hipEventRecord(ds->join[g], gs[g]) != hipSuccess) return PF_ELAUNCH;
            if (hipStreamWaitEvent(s, ds->join[g], 0) != hipSuccess) return PF_ELAUNCH;
        }
        return PF_OK;
    }

    // One step of group g: the (chunk, layer) pairs of one diagonal.  Per step:
    // quantise the layer inputs (rebuilding them from the previous down
    // product's split partials on the skinny path), the six K = H products,
    // quantise up, the down product.  `fin` carries the chunk whose last down
    // product ran in the previous step; its rows are rebuilt without
    // quantisation into the output.  step == group_steps(g) only finalises.
    // chunks of group g active at `step` (each at layer step - start)
    std::vector<int64_t> active(int g, int64_t step) const
    {
        std::vector<int64_t> cs;
        const int64_t K = group_chunks(g);
        if (step >= 0 && step < group_steps(g))
            for (int64_t k = 0; k < K && start(k) <= step; ++k)
                if (start(k) + L() > step) cs.push_back(g + k * ng);
        return cs;
    }

    // The attention of the (chunk, layer) pairs group g ran at `step`: each
    // token over the cache positions up to its own, quantised, then the o
    // product.  Every earlier chunk's rows of the same layer are in the cache
    // once every group has finished its step-`step` products (a chunk never
    // reaches a layer before an earlier chunk of any group), which the
    // per-group step marks establish.
    pf_status attention_of(Recorder& rec, int g, int64_t step, hipStream_t sg)
    {
        const std::vector<int64_t> cs = active(g, step);
        if (cs.empty()) return PF_OK;
        if (ng > 1)
            for (int o = 0; o < ng; ++o)
                if (o != g && hipStreamWaitEvent(sg, ds->kvdone[o][step & 1], 0) != hipSuccess)
                    return PF_ELAUNCH;
        const bool skinny = ch <= 64;
        AttnStep A;
        std::memset(&A, 0, sizeof(A));
        A.H = (int)H();
        A.n_heads = (int)st->n_heads;
        A.d = (int)(H() / st->n_heads);
        A.scale = 1.0f / sqrtf((float)A.d);
        A.ldq = NT();
        A.ldkv = H();
        StackStep O;
        std::memset(&O, 0, sizeof(O));
        O.nproj = 1;
        O.K = (int)H();
        O.rows[0] = (int)H();
        O.yoff[0] = (int)offs(3);
        const int tm = (int)((ch + tiled_tokens(ch) - 1) / tiled_tokens(ch));
        O.tiles_m = tm;
        O.tile_off[1] = (int)(skinny ? (H() + kSkinnyRows - 1) / kSkinnyRows
                                     : ((H() + kTiledRows - 1) / kTiledRows) * tm);
        O.splits = 1;
        O.kb_per_split = (int)(H() / 64);
        O.ldx = H();
        O.ldy = NT();
        O.kv_proj[0] = O.kv_proj[1] = -1;
        O.nostore = proj ? 0u : 1u;                      // o's rows feed nothing further
        double a_bytes = 0, o_bytes = 0;
        for (int64_t c : cs) {
            const int64_t l = step - start(c / ng), c0 = c * ch, M = std::min(ch, P - c0);
            char* sl = slot(c);
            AttnPair& ap = A.pair[A.npairs++];
            ap.q = rows(c, l) + offs(0);
            ap.K = kv_rows(l, 0, 0);
            ap.V = kv_rows(l, 1, 0);
            ap.ao = reinterpret_cast<int8_t*>(sl + lay.ao);
            ap.sao = reinterpret_cast<float*>(sl + lay.sao);
            ap.pos0 = (int)c0;
            ap.M = (int)M;
            A.max_m = std::max(A.max_m, (int)M);
            // q read, the K/V history once, codes and scales written
            a_bytes += (double)M * H() * 4 + 2.0 * (c0 + M) * H() * 4 + (double)M * H() + 4.0 * M;
            StepPair& po = O.pair[O.npairs++];
            const pf_layer& ly = layer(c, l);
            po.W[0] = ly.W[3];
            po.ws[0] = ly.w_scale[3];
            po.X = ap.ao;
            po.xs = ap.sao;
            po.Y = rows(c, l);
            po.M = (int)M;
            o_bytes += product_bytes(H(), H(), M);
        }
        pf_status r = rec.run(Recorder::kAttn, a_bytes, [&] { return launched(launch_attention(A, sg)); });
        if (r) return r;
        const int tb = (int)((ch + 15) / 16);
        return rec.run(Recorder::kProduct, o_bytes, [&] {
            if (!skinny) return launched(launch_gemm_tiled_step(O, ch, sg));
            return launched(H() / 64 <= 16 ? launch_gemm_xres(O, tb, sg) : launch_gemm_stream(O, tb, sg));
        });
    }

    pf_status group_step(Recorder& rec, int g, int64_t step, int64_t& fin, hipStream_t sg)
    {
        const int64_t L = this->L();
        const bool skinny = ch <= 64;
        // the attention of the previous step's pairs (their q rows are intact:
        // this step's products have not run yet on this stream)
        if (attn())
            if (pf_status r = attention_of(rec, g, step - 1, sg)) return r;
        // token-resident kernel for the six K = H products when a split of H fits
        const bool xres_a = skinny && H() / 64 <= 16;
        const int sd = lay.dsplits;
        // the down product leaves int32 split partials that the next
        // quantisation launch sums (always on the skinny path)
        const bool rebuild_d = skinny || sd > 1;
        // the K = H products of the step: q, k, v, o, gate, up; with attention o
        // waits for it and the launch has five
        const int projA6[6] = {0, 1, 2, 3, 4, 5}, projA5[6] = {0, 1, 2, 4, 5, 5};
        const int* projA = attn() ? projA5 : projA6;
        const int nA = attn() ? 5 : 6;
        int64_t rowsA[6];
        for (int j = 0; j < 6; ++j) rowsA[j] = projA[j] >= 4 ? F() : H();
        const int tm = (int)((ch + tiled_tokens(ch) - 1) / tiled_tokens(ch));
        const int tb = (int)((ch + 15) / 16);
        const std::vector<int64_t> cs = active(g, step);   // global chunk indices active in this step
        QuantStep qa, qd;
        StackStep A, D;
        std::memset(&qa, 0, sizeof(qa));
        std::memset(&qd, 0, sizeof(qd));
        std::memset(&A, 0, sizeof(A));
        std::memset(&D, 0, sizeof(D));
        qa.K = (int)H();
        qd.K = (int)F();
        A.nproj = nA;
        A.K = (int)H();
        A.splits = 1;
        A.kb_per_split = (int)(H() / 64);
        D.nproj = 1;
        D.K = (int)F();
        D.splits = sd;
        D.partials = rebuild_d ? 1 : 0;
        D.kb_per_split = lay.dkb;
        A.tiles_m = D.tiles_m = tm;
        A.ldx = H();
        D.ldx = F();
        A.ldy = D.ldy = NT();
        D.ldy2 = H();
        D.ldp = H();
        D.part_stride = ch * H();
        // with attention, k and v (slots 1 and 2 of the launch) also go to the cache
        A.kv_proj[0] = attn() ? 1 : -1;
        A.kv_proj[1] = attn() ? 2 : -1;
        A.ldkv = H();
        A.nostore = unread_rows(projA, nA);
        D.kv_proj[0] = D.kv_proj[1] = -1;
        for (int j = 0; j < nA; ++j) {
            A.rows[j] = (int)rowsA[j];
            A.yoff[j] = (int)offs(projA[j]);
            const int64_t t = skinny ? (rowsA[j] + kSkinnyRows - 1) / kSkinnyRows
                                     : ((rowsA[j] + kTiledRows - 1) / kTiledRows) * tm;
            A.tile_off[j + 1] = A.tile_off[j] + (int)t;
        }
        D.rows[0] = (int)H();
        D.yoff[0] = (int)offs(6);
        D.tile_off[1] = (int)(skinny ? (H() + kSkinnyRows - 1) / kSkinnyRows : ((H() + kTiledRows - 1) / kTiledRows) * tm);
        double qa_bytes = 0, qd_bytes = 0, a_bytes = 0, d_bytes = 0, part_bytes = 0;
        int rows_a = 0, rows_d = 0;
        auto rebuild = [&](QuantPair& q, int64_t c, int64_t l_prev, bool last) {
            // rows of (c, l_prev)'s down product, from its split partials
            char* sl = slot(c);
            q.part = reinterpret_cast<const int*>(sl + lay.part);
            q.part_stride = ch * H();
            q.splits = sd;
            q.ws = layer(c, l_prev).w_scale[6];
            q.as = reinterpret_cast<const float*>(sl + lay.sb);
            // the rebuilt f32 rows: kept only for the caller's projection rows
            // (the codes come from registers), or where the quantisation reads
            // them back (rows of more than 16384 values)
            q.h = (proj || H() > 16384) ? rows(c, l_prev) + offs(6) : nullptr;
            q.ldh = NT();
            q.y = last ? y + c * ch * H() : nullptr;
        };
        for (size_t i = 0; i < cs.size(); ++i) {
            const int64_t c = cs[i], l = step - start(c / ng);
            const int64_t c0 = c * ch, M = std::min(ch, P - c0);
            const pf_layer& ly = layer(c, l);
            char* sl = slot(c);
            int8_t* a = reinterpret_cast<int8_t*>(sl + lay.a);
            int8_t* b = reinterpret_cast<int8_t*>(sl + lay.b);
            float* sa = reinterpret_cast<float*>(sl + lay.sa);
            float* sb = reinterpret_cast<float*>(sl + lay.sb);
            float* out = rows(c, l);
            QuantPair& q0 = qa.pair[qa.npairs++];
            if (l == 0) {
                q0.src = x + c0 * H();
                q0.ld = H();
            } else if (rebuild_d) {
                rebuild(q0, c, l - 1, false);
                part_bytes += (double)M * H() * 4 * sd;       // the partials' re-read
            } else {
                q0.src = rows(c, l - 1) + offs(6);
                q0.ld = NT();
            }
            q0.q = a;
            q0.s = sa;
            q0.row0 = rows_a;
            rows_a += (int)M;
            QuantPair& q1 = qd.pair[qd.npairs++];
            q1.src = out + offs(5);
            q1.gate = st->activation == PF_ACT_SWIGLU ? out + offs(4) : nullptr;
            q1.ld = NT();
            q1.q = b;
            q1.s = sb;
            q1.row0 = rows_d;
            rows_d += (int)M;
            StepPair& pa = A.pair[A.npairs++];
            // the products share one read of the quantised tokens
            a_bytes += (double)M * H() + 4.0 * M;
            for (int j = 0; j < nA; ++j) {
                pa.W[j] = ly.W[projA[j]];
                pa.ws[j] = ly.w_scale[projA[j]];
                a_bytes += weight_out_bytes(rowsA[j], H(), M);
            }
            if (attn()) {
                pa.kv[0] = kv_rows(l, 0, c0);
                pa.kv[1] = kv_rows(l, 1, c0);
            }
            pa.X = a;
            pa.xs = sa;
            pa.Y = out;
            pa.M = (int)M;
            StepPair& pd = D.pair[D.npairs++];
            pd.W[0] = ly.W[6];
            pd.ws[0] = ly.w_scale[6];
            pd.X = b;
            pd.xs = sb;
            pd.Y = out;
            pd.Y2 = (!rebuild_d && l == L - 1) ? y + c0 * H() : nullptr;
            pd.part = reinterpret_cast<int*>(sl + lay.part);
            pd.M = (int)M;
            d_bytes += product_bytes(H(), F(), M);
            if (rebuild_d) part_bytes += (double)M * H() * 4 * sd;   // the partials' write
            qa_bytes += (double)M * H() * 5 + M * 4.0;
            // up read (and gate with the gated SiLU), codes and scales written
            qd_bytes += (double)M * F() * (st->activation == PF_ACT_SWIGLU ? 9 : 5) + M * 4.0;
        }
        if (fin >= 0) {
            // the chunk that left the last layer: rebuild its output, no quantisation
            const int64_t M = std::min(ch, P - fin * ch);
            QuantPair& qf = qa.pair[qa.npairs++];
            rebuild(qf, fin, L - 1, true);
            qf.row0 = rows_a;
            rows_a += (int)M;
            // completes the last down product's epilogue: its output bytes are
            // the product's; the partials' re-read is overhead
            part_bytes += (double)M * H() * 4 * sd;
            fin = -1;
        }
        qa.total_rows = rows_a;
        qd.total_rows = rows_d;
        pf_status r = PF_OK;
        if (qa.npairs > 0)
            r = rec.run(Recorder::kQuant, qa_bytes, [&] { return launched(launch_quantize_step(qa, sg)); }, sg);
        if (r) return r;
        if (cs.empty()) {
            rec.overhead(part_bytes);
            if (attn() && ng > 1 && hipEventRecord(ds->kvdone[g][step & 1], sg) != hipSuccess)
                return PF_ELAUNCH;
            return PF_OK;
        }
        r = rec.run(Recorder::kProduct, a_bytes, [&] {
            if (!skinny) return launched(launch_gemm_tiled_step(A, ch, sg));
            return launched(xres_a ? launch_gemm_xres(A, tb, sg) : launch_gemm_stream(A, tb, sg));
        }, sg);
        // this step's cache rows are written once the products above are done
        if (!r && attn() && ng > 1 && hipEventRecord(ds->kvdone[g][step & 1], sg) != hipSuccess)
            return PF_ELAUNCH;
        if (!r) r = rec.run(Recorder::kQuant, qd_bytes,
                            [&] { return launched(launch_quantize_step(qd, sg)); }, sg);
        if (!r) r = rec.run(Recorder::kProduct, d_bytes, [&] {
            return launched(skinny ? launch_gemm_xres(D, tb, sg) : launch_gemm_tiled_step(D, ch, sg));
        }, sg);
        if (r) return r;
        rec.overhead(part_bytes);
        if (rebuild_d)
            for (int64_t c : cs)
                if (step - start(c / ng) == L - 1) fin = c;
        return PF_OK;
    }

    pf_status per_token(Recorder& rec)
    {
        const int64_t L = st->n_layers;
        char* sl = slot(0);
        int8_t* a = reinterpret_cast<int8_t*>(sl + lay.a);
        int8_t* b = reinterpret_cast<int8_t*>(sl + lay.b);
        float* sa = reinterpret_cast<float*>(sl + lay.sa);
        float* sb = reinterpret_cast<float*>(sl + lay.sb);
        float* scratch = reinterpret_cast<float*>(sl + lay.proj);
        const int64_t rowsA[6] = {H(), H(), H(), H(), F(), F()};
        char* none = nullptr;
        for (int64_t t = 0; t < P; ++t) {
            for (int64_t l = 0; l < L; ++l) {
                const pf_layer& ly = st->layers[l];
                float* out = proj ? proj + ((size_t)l * P + t) * NT() : scratch;
                const float* hin = l == 0 ? x + t * H()
                                          : (proj ? proj + ((size_t)(l - 1) * P + t) * NT() : scratch) + offs(6);
                pf_status r = rec.run(Recorder::kQuant, (double)H() * 5 + 4, [&] {
                    return launched(launch_quantize(hin, H(), 1, (int)H(), a, sa, s));
                });
                if (r) return r;
                GemmSet set;
                std::memset(&set, 0, sizeof(set));
                double bytes = (double)H() + 4.0;        // the token, read once
                for (int j = 0; j < 6; ++j) {
                    if (attn() && j == 3) continue;      // o waits for the attention
                    GemmProb& gp = set.p[set.nprob++];
                    make_skinny(gp, ly.W[j], ly.w_scale[j], rowsA[j], H(), a, H(), sa, 1,
                                out + offs(j), NT(), unsplit(rowsA[j], H()), none, 1);
                    if (attn() && (j == 1 || j == 2)) gp.Y2 = kv_rows(l, j - 1, t);   // the cache
                    bytes += weight_out_bytes(rowsA[j], H(), 1);
                }
                finish_set(set, 0);
                r = rec.run(Recorder::kProduct, bytes, [&] { return launched(launch_gemv(set, s)); });
                if (r) return r;
                if (attn()) {
                    // token t over cache positions 0 .. t of layer l, then o
                    AttnStep A;
                    std::memset(&A, 0, sizeof(A));
                    A.H = (int)H();
                    A.n_heads = (int)st->n_heads;
                    A.d = (int)(H() / st->n_heads);
                    A.scale = 1.0f / sqrtf((float)A.d);
                    A.ldq = NT();
                    A.ldkv = H();
                    A.npairs = 1;
                    A.max_m = 1;
                    AttnPair& ap = A.pair[0];
                    ap.q = out + offs(0);
                    ap.K = kv_rows(l, 0, 0);
                    ap.V = kv_rows(l, 1, 0);
                    ap.ao = reinterpret_cast<int8_t*>(sl + lay.ao);
                    ap.sao = reinterpret_cast<float*>(sl + lay.sao);
                    ap.pos0 = (int)t;
                    ap.M = 1;
                    r = rec.run(Recorder::kAttn, (double)H() * 4 * (1 + 2 * (t + 1)) + H() + 4.0,
                                [&] { return launched(launch_attention(A, s)); });
                    if (r) return r;
                    GemmSet os;
                    std::memset(&os, 0, sizeof(os));
                    os.nprob = 1;
                    make_skinny(os.p[0], ly.W[3], ly.w_scale[3], H(), H(), ap.ao, H(), ap.sao, 1,
                                out + offs(3), NT(), unsplit(H(), H()), none, 1);
                    finish_set(os, 0);
                    r = rec.run(Recorder::kProduct, product_bytes(H(), H(), 1),
                                [&] { return launched(launch_gemv(os, s)); });
                    if (r) return r;
                }
                const bool gated = st->activation == PF_ACT_SWIGLU;
                r = rec.run(Recorder::kQuant, (double)F() * (gated ? 9 : 5) + 4, [&] {
                    if (gated)
                        return launched(launch_quantize_gated(out + offs(5), out + offs(4), NT(), 1,
                                                              (int)F(), b, sb, s));
                    return launched(launch_quantize(out + offs(5), NT(), 1, (int)F(), b, sb, s));
                });
                if (r) return r;
                GemmSet dn;
                std::memset(&dn, 0, sizeof(dn));
                dn.nprob = 1;
                make_skinny(dn.p[0], ly.W[6], ly.w_scale[6], H(), F(), b, F(), sb, 1, out + offs(6),
                            NT(), unsplit(H(), F()), none, 1);
                if (l == L - 1) {
                    dn.p[0].Y2 = y + t * H();
                    dn.p[0].ldy2 = H();
                }
                finish_set(dn, 0);
                r = rec.run(Recorder::kProduct, product_bytes(H(), F(), 1),
                            [&] { return launched(launch_gemv(dn, s)); });
                if (r) return r;
            }
        }
        return PF_OK;
    }
};

// 65 to 128 tokens: products of at most this many weight bytes go through the
// token-resident kernel (eight 16-token blocks, K split into slices of at most
// 8 k-blocks) instead of the tiled one, whose 256-row tiles are then too few.
constexpr int64_t kXres128MaxBytes = 16 << 20;

bool xres128(int64_t N, int64_t K, int64_t M)
{
    return M > 64 && M <= 128 && N * K <= kXres128MaxBytes;
}

SkinnyPlan plan_xres128(int64_t N, int64_t K)
{
    SkinnyPlan p = unsplit(N, K);
    const int nkb = (int)(K / 64);
    p.kb_per_split = std::min(nkb, xres_max_kb(8));
    p.splits = (nkb + p.kb_per_split - 1) / p.kb_per_split;
    return p;
}


// Argument checks of a chunk product (M = 0 passes: a no-op).
pf_status check_chunk_args(const int8_t* W, const float* w_scale, int64_t N, int64_t K,
                           const int8_t* xq, const float* a_scale, int64_t M, const float* y)
{
    if (N <= 0 || N > INT32_MAX || !valid_k(K) || M < 0 || M > INT32_MAX) return PF_EINVAL;
    // the tiled kernel addresses a matrix by 32-bit offsets
    if ((uint64_t)N * (uint64_t)K >= (1ull << 32) || (uint64_t)M * (uint64_t)K >= (1ull << 32)) return PF_EINVAL;
    if (M == 0) return PF_OK;
    if (!W || !w_scale || !xq || !a_scale || !y) return PF_EINVAL;
    if (!aligned16(W) || !aligned4(w_scale) || !aligned16(xq) || !aligned4(a_scale) || !aligned4(y))
        return PF_EINVAL;
    const size_t yb = (size_t)M * N * 4;
    if (overlap(y, yb, W, (size_t)N * K) || overlap(y, yb, w_scale, (size_t)N * 4) ||
        overlap(y, yb, xq, (size_t)M * K) || overlap(y, yb, a_scale, (size_t)M * 4))
        return PF_EINVAL;
    return PF_OK;
}

// Scratch bytes a chunk product's plan uses when room to split is given (0:
// it runs unsplit).
size_t chunk_scratch_bytes(int64_t N, int64_t K, int64_t M, const float* y)
{
    if (M <= 64) return split_bytes(N, M, plan_chunk_small(N, K, xres_fits_shape(N, y)));
    if (xres128(N, K, M) && xres_fits_shape(N, y)) return split_bytes(N, M, plan_xres128(N, K));
    return split_bytes(N, M, plan_tiled(N, K, M));
}

// A validated chunk product (M > 0) on a gfx950 device: the plan by M, split
// across workgroups when the workspace has room for the split's partials.
pf_status run_chunk(const int8_t* W, const float* w_scale, int64_t N, int64_t K, const int8_t* xq,
                    const float* a_scale, int64_t M, float* y, void* workspace, size_t ws_bytes,
                    hipStream_t stream)
{
    GemmSet set;
    std::memset(&set, 0, sizeof(set));
    set.nprob = 1;
    int tile_tokens = 0;
    char* scratch = static_cast<char*>(workspace);
    if (M <= 64) {
        SkinnyPlan p = plan_chunk_small(N, K, xres_fits_shape(N, y));
        if (!workspace || ws_bytes < split_bytes(N, M, p)) p = unsplit(N, K);
        make_skinny(set.p[0], W, w_scale, N, K, xq, K, a_scale, M, y, N, p, scratch, M);
    } else if (xres128(N, K, M) && xres_fits_shape(N, y) &&
               (plan_xres128(N, K).splits == 1 ||
                (workspace && ws_bytes >= split_bytes(N, M, plan_xres128(N, K))))) {
        const SkinnyPlan p = plan_xres128(N, K);
        make_skinny(set.p[0], W, w_scale, N, K, xq, K, a_scale, M, y, N, p, scratch, M);
        return run_skinny_xres(set, M, stream);
    } else {
        SkinnyPlan p = plan_tiled(N, K, M);
        if (!workspace || ws_bytes < split_bytes(N, M, p)) p = plan_tiled(N, K, M, 1);
        make_tiled(set.p[0], W, w_scale, N, K, xq, K, a_scale, M, y, N, p, scratch);
        tile_tokens = p.tokens;
    }
    return run_products(set, M, tile_tokens, stream);
}


// ---------------------------------------------------------------------------
// Scratch of pf_gemm_i8_chunk_noalloc: the split partials live in this
// file-scope device array instead of a caller's workspace.  Each device holds
// its own copy at its own address, looked up once per device at set-up (the
// array's name in host code is not a device address).
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
__device__ __attribute__((aligned(256))) char scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[64];

// The device address of this device's scratch array (null if the lookup fails).
void* scratch_ptr()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return nullptr;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}


// ---------------------------------------------------------------------------
// The stack with its weights in host memory ("Predictive prefetch": the
// weights of layer L + 1 are copied into the other buffer of a ring while
// layer L computes; "Single-pass prefill": every prompt position goes through
// a layer while its weights are loaded, so each layer crosses the host link
// once per prompt).  Device ring of n_buffers layer slots, fed by a copy
// stream; the compute stream waits for layer l's copy only before its first
// product, and the copy of layer l into a slot waits for the compute that last
// used the slot.

// One layer's weights and scales in a ring slot.
struct SlotLayout {
    size_t w[PF_NPROJ], s[PF_NPROJ], bytes;
};

SlotLayout slot_layout(int64_t H, int64_t F)
{
    const int64_t rows[PF_NPROJ] = {H, H, H, H, F, F, H};
    const int64_t cols[PF_NPROJ] = {H, H, H, H, H, H, F};
    SlotLayout S{};
    size_t o = 0;
    for (int j = 0; j < PF_NPROJ; ++j) {
        S.w[j] = o;
        o += round_up((size_t)rows[j] * cols[j], kAlign);
    }
    for (int j = 0; j < PF_NPROJ; ++j) {
        S.s[j] = o;
        o += round_up((size_t)rows[j] * 4, kAlign);
    }
    S.bytes = o;
    return S;
}

// Workspace of the streamed stack: the ring, then the prompt's activations for
// the layer in flight: codes a [P][H] and b [P][F] with scales, and the
// projection rows [P][5H + 2F] (the down column is the next layer's input).
struct StreamLayout {
    SlotLayout sl;
    size_t ring, a, b, sa, sb, rows, total;
};

StreamLayout stream_layout(int64_t H, int64_t F, int64_t P, int64_t nbuf)
{
    StreamLayout S{};
    S.sl = slot_layout(H, F);
    size_t o = 0;
    S.ring = o; o += S.sl.bytes * (size_t)nbuf;
    S.a = o; o += round_up((size_t)P * H, kAlign);
    S.b = o; o += round_up((size_t)P * F, kAlign);
    S.sa = o; o += round_up((size_t)P * 4, kAlign);
    S.sb = o; o += round_up((size_t)P * 4, kAlign);
    S.rows = o; o += round_up((size_t)P * (5 * H + 2 * F) * 4, kAlign);
    S.total = o;
    return S;
}

struct StreamRun {
    const pf_stack* st;
    const float* x;
    int64_t P, ch, nbuf;
    float* y;
    char* ws;
    StreamLayout lay;
    hipStream_t s, cs;
    std::vector<hipEvent_t> copied, computed;   // per layer, timing events

    ~StreamRun()
    {
        for (hipEvent_t e : copied) if (e) (void)hipEventDestroy(e);
        for (hipEvent_t e : computed) if (e) (void)hipEventDestroy(e);
    }
    int64_t H() const { return st->hidden; }
    int64_t F() const { return st->ffn; }
    int64_t NT() const { return 5 * st->hidden + 2 * st->ffn; }
    int64_t offs(int j) const
    {
        const int64_t o[PF_NPROJ] = {0, H(), 2 * H(), 3 * H(), 4 * H(), 4 * H() + F(), 4 * H() + 2 * F()};
        return o[j];
    }
    char* slot(int64_t l) const { return ws + lay.ring + (size_t)(l % nbuf) * lay.sl.bytes; }
    float* rows() const { return reinterpret_cast<float*>(ws + lay.rows); }

    // layer l's weights host -> its ring slot, on the copy stream
    pf_status copy_layer(int64_t l)
    {
        const int64_t H = this->H(), F = this->F();
        const int64_t rws[PF_NPROJ] = {H, H, H, H, F, F, H};
        const int64_t cls[PF_NPROJ] = {H, H, H, H, H, H, F};
        if (l >= nbuf && hipStreamWaitEvent(cs, computed[l - nbuf], 0) != hipSuccess) return PF_ELAUNCH;
        char* sl = slot(l);
        const pf_layer& ly = st->layers[l];
        for (int j = 0; j < PF_NPROJ; ++j) {
            if (hipMemcpyAsync(sl + lay.sl.w[j], ly.W[j], (size_t)rws[j] * cls[j], hipMemcpyHostToDevice, cs) !=
                    hipSuccess ||
                hipMemcpyAsync(sl + lay.sl.s[j], ly.w_scale[j], (size_t)rws[j] * 4, hipMemcpyHostToDevice, cs) !=
                    hipSuccess)
                return launched(hipGetLastError());
        }
        return hipEventRecord(copied[l], cs) == hipSuccess ? PF_OK : PF_ELAUNCH;
    }

    // every chunk of the prompt through layer l (weights in its slot)
    pf_status compute_layer(int64_t l)
    {
        const int64_t H = this->H(), F = this->F(), L = st->n_layers;
        char* sl = slot(l);
        int8_t* a = reinterpret_cast<int8_t*>(ws + lay.a);
        int8_t* b = reinterpret_cast<int8_t*>(ws + lay.b);
        float* sa = reinterpret_cast<float*>(ws + lay.sa);
        float* sb = reinterpret_cast<float*>(ws + lay.sb);
        float* R = rows();
        // quantise the layer input of every token (x, or the previous down)
        QuantStep q;
        std::memset(&q, 0, sizeof(q));
        q.npairs = 1;
        q.K = (int)H;
        q.total_rows = (int)P;
        q.pair[0].src = l == 0 ? x : R + offs(6);
        q.pair[0].ld = l == 0 ? H : NT();
        q.pair[0].q = a;
        q.pair[0].s = sa;
        if (pf_status r = launched(launch_quantize_step(q, s))) return r;
        if (hipStreamWaitEvent(s, copied[l], 0) != hipSuccess) return PF_ELAUNCH;
        const bool skinny = ch <= 64;
        const int tb = (int)((ch + 15) / 16);
        const int tm = (int)((ch + tiled_tokens(ch) - 1) / tiled_tokens(ch));
        const int64_t rowsA[6] = {H, H, H, H, F, F};
        const int64_t C = (P + ch - 1) / ch;
        auto wptr = [&](int j) { return reinterpret_cast<const int8_t*>(sl + lay.sl.w[j]); };
        auto sptr = [&](int j) { return reinterpret_cast<const float*>(sl + lay.sl.s[j]); };
        // the six K = H products, chunks as the pairs of a launch
        for (int64_t c0 = 0; c0 < C; c0 += kMaxPairs) {
            StackStep A;
            std::memset(&A, 0, sizeof(A));
            A.nproj = 6;
            A.K = (int)H;
            A.splits = 1;
            A.kb_per_split = (int)(H / 64);
            A.tiles_m = tm;
            A.ldx = H;
            A.ldy = NT();
            A.kv_proj[0] = A.kv_proj[1] = -1;
            // q, k, v and o feed nothing here, gate only the gated SiLU: their
            // rows are not stored
            A.nostore = st->activation == PF_ACT_SWIGLU ? 0x0fu : 0x1fu;
            for (int j = 0; j < 6; ++j) {
                A.rows[j] = (int)rowsA[j];
                A.yoff[j] = (int)offs(j);
                const int64_t t = skinny ? (rowsA[j] + kSkinnyRows - 1) / kSkinnyRows
                                         : ((rowsA[j] + kTiledRows - 1) / kTiledRows) * tm;
                A.tile_off[j + 1] = A.tile_off[j] + (int)t;
            }
            for (int64_t c = c0; c < std::min(C, c0 + kMaxPairs); ++c) {
                const int64_t t0 = c * ch, M = std::min(ch, P - t0);
                StepPair& p = A.pair[A.npairs++];
                for (int j = 0; j < 6; ++j) {
                    p.W[j] = wptr(j);
                    p.ws[j] = sptr(j);
                }
                p.X = a + t0 * H;
                p.xs = sa + t0;
                p.Y = R + t0 * NT();
                p.M = (int)M;
            }
            pf_status r;
            if (!skinny) r = launched(launch_gemm_tiled_step(A, ch, s));
            else r = launched(H / 64 <= 16 ? launch_gemm_xres(A, tb, s) : launch_gemm_stream(A, tb, s));
            if (r) return r;
        }
        // the down product's input: up, or silu(gate) * up
        QuantStep qd;
        std::memset(&qd, 0, sizeof(qd));
        qd.npairs = 1;
        qd.K = (int)F;
        qd.total_rows = (int)P;
        qd.pair[0].src = R + offs(5);
        qd.pair[0].gate = st->activation == PF_ACT_SWIGLU ? R + offs(4) : nullptr;
        qd.pair[0].ld = NT();
        qd.pair[0].q = b;
        qd.pair[0].s = sb;
        if (pf_status r = launched(launch_quantize_step(qd, s))) return r;
        // down, whole K per tile (no split partials), the last layer also to y
        for (int64_t c0 = 0; c0 < C; c0 += kMaxPairs) {
            StackStep D;
            std::memset(&D, 0, sizeof(D));
            D.nproj = 1;
            D.K = (int)F;
            D.splits = 1;
            D.kb_per_split = (int)(F / 64);
            D.tiles_m = tm;
            D.ldx = F;
            D.ldy = NT();
            D.ldy2 = H;
            D.kv_proj[0] = D.kv_proj[1] = -1;
            D.rows[0] = (int)H;
            D.yoff[0] = (int)offs(6);
            D.tile_off[1] = (int)(skinny ? (H + kSkinnyRows - 1) / kSkinnyRows
                                         : ((H + kTiledRows - 1) / kTiledRows) * tm);
            for (int64_t c = c0; c < std::min(C, c0 + kMaxPairs); ++c) {
                const int64_t t0 = c * ch, M = std::min(ch, P - t0);
                StepPair& p = D.pair[D.npairs++];
                p.W[0] = wptr(6);
                p.ws[0] = sptr(6);
                p.X = b + t0 * F;
                p.xs = sb + t0;
                p.Y = R + t0 * NT();
                p.Y2 = l == L - 1 ? y + t0 * H : nullptr;
                p.M = (int)M;
            }
            pf_status r = launched(skinny ? launch_gemm_stream(D, tb, s) : launch_gemm_tiled_step(D, ch, s));
            if (r) return r;
        }
        return hipEventRecord(computed[l], s) == hipSuccess ? PF_OK : PF_ELAUNCH;
    }

    pf_status run()
    {
        const int64_t L = st->n_layers;
        copied.assign((size_t)L, nullptr);
        computed.assign((size_t)L, nullptr);
        for (int64_t l = 0; l < L; ++l)
            if (hipEventCreate(&copied[l]) != hipSuccess || hipEventCreate(&computed[l]) != hipSuccess)
                return PF_ELAUNCH;
        // the copy stream starts after the caller's earlier work (the ring may
        // hold a previous call's layers)
        hipEvent_t fork = nullptr;
        if (hipEventCreateWithFlags(&fork, hipEventDisableTiming) != hipSuccess) return PF_ELAUNCH;
        pf_status r = hipEventRecord(fork, s) == hipSuccess && hipStreamWaitEvent(cs, fork, 0) == hipSuccess
                          ? PF_OK : PF_ELAUNCH;
        (void)hipEventDestroy(fork);
        // copies run up to nbuf - 1 layers ahead of the compute
        for (int64_t l = 0; l < std::min(nbuf - 1, L) && !r; ++l) r = copy_layer(l);
        for (int64_t l = 0; l < L && !r; ++l) {
            if (l + nbuf - 1 < L) r = copy_layer(l + nbuf - 1);
            if (!r) r = compute_layer(l);
        }
        return r;
    }
};

}  // namespace

// ===========================================================================
extern "C" {

const char* pf_status_string(pf_status s)
{
    switch (s) {
        case PF_OK: return "PF_OK";
        case PF_EINVAL: return "PF_EINVAL: invalid argument";
        case PF_ENODEV: return "PF_ENODEV: no gfx950 device is current";
        case PF_ELAUNCH: return "PF_ELAUNCH: a HIP launch failed";
        case PF_EWORKSPACE: return "PF_EWORKSPACE: workspace missing or too small";
        case PF_EINTERNAL: return "PF_EINTERNAL: internal error";
        default: return "unknown pf_status";
    }
}

pf_status pf_init(void)
{
    try {
        if (pf_status st = check_device()) return st;
        return scratch_ptr() ? PF_OK : PF_ELAUNCH;
    } catch (...) {
        return PF_EINTERNAL;
    }
}

pf_status pf_workspace_clear(void* workspace, size_t bytes, void* stream)
{
    try {
        if (bytes == 0) return PF_OK;
        if (!workspace || !aligned16(workspace)) return PF_EINVAL;
        if (pf_status st = check_device()) return st;
        return launched(launch_fill_zero(workspace, bytes, (hipStream_t)stream));
    } catch (...) {
        return PF_EINTERNAL;
    }
}

pf_status pf_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* xq,
                          float* a_scale, void* stream)
{
    try {
        if (M < 0 || K <= 0 || K % 4 != 0 || ldx < K || ldx % 4 != 0 || M > INT32_MAX)
            return PF_EINVAL;
        if (M == 0) return PF_OK;
        if (!x || !xq || !a_scale || !aligned16(x) || !aligned16(xq) || !aligned4(a_scale))
            return PF_EINVAL;
        const size_t xb = (size_t)((M - 1) * ldx + K) * 4;
        if (overlap(x, xb, xq, (size_t)M * K) || overlap(x, xb, a_scale, (size_t)M * 4) ||
            overlap(xq, (size_t)M * K, a_scale, (size_t)M * 4))
            return PF_EINVAL;
        if (pf_status st = check_device()) return st;
        return launched(launch_quantize(x, ldx, (int)M, (int)K, xq, a_scale, (hipStream_t)stream));
    } catch (...) {
        return PF_EINTERNAL;
    }
}

size_t pf_gemm_i8_chunk_workspace(int64_t N, int64_t K, int64_t M)
{
    if (N <= 0 || N > INT32_MAX || !valid_k(K) || M <= 0 || M > INT32_MAX) return 0;
    if (M > 64) {
        const size_t tiled = split_bytes(N, M, plan_tiled(N, K, M));
        return xres128(N, K, M) ? std::max(tiled, split_bytes(N, M, plan_xres128(N, K))) : tiled;
    }
    // the output's alignment picks the plan: room for either
    return std::max(split_bytes(N, M, plan_chunk_small(N, K, true)),
                    split_bytes(N, M, plan_chunk_small(N, K, false)));
}

pf_status pf_gemm_i8_chunk(const int8_t* W, const float* w_scale, int64_t N, int64_t K,
                           const int8_t* xq, const float* a_scale, int64_t M, float* y,
                           void* workspace, size_t ws_bytes, void* stream)
{
    try {
        if (pf_status st = check_chunk_args(W, w_scale, N, K, xq, a_scale, M, y)) return st;
        if (M == 0) return PF_OK;
        if (workspace && !aligned16(workspace)) return PF_EINVAL;
        if (workspace && overlap(workspace, ws_bytes, y, (size_t)M * N * 4)) return PF_EINVAL;
        if (pf_status st = check_device()) return st;
        return run_chunk(W, w_scale, N, K, xq, a_scale, M, y, workspace, ws_bytes,
                         (hipStream_t)stream);
    } catch (...) {
        return PF_EINTERNAL;
    }
}

pf_status pf_gemm_i8_chunk_noalloc(const int8_t* W, const float* w_scale, int64_t N, int64_t K,
                                   const int8_t* xq, const float* a_scale, int64_t M, float* y,
                                   void* stream)
{
    try {
        if (pf_status st = check_chunk_args(W, w_scale, N, K, xq, a_scale, M, y)) return st;
        if (M == 0) return PF_OK;
        if (chunk_scratch_bytes(N, K, M, y) > kNoallocScratchBytes) return PF_EWORKSPACE;
        if (pf_status st = check_device()) return st;
        void* ws = scratch_ptr();
        if (!ws) return PF_ELAUNCH;
        return run_chunk(W, w_scale, N, K, xq, a_scale, M, y, ws, kNoallocScratchBytes,
                         (hipStream_t)stream);
    } catch (...) {
        return PF_EINTERNAL;
    }
}

pf_status pf_gemv_i8(const int8_t* W, const float* w_scale, int64_t N, int64_t K,
                     const int8_t* xq, const float* a_scale, float* y, void* stream)
{
    try {
        if (N <= 0 || N > INT32_MAX || !valid_k(K)) return PF_EINVAL;
        if (!W || !w_scale || !xq || !a_scale || !y) return PF_EINVAL;
        if (!aligned16(W) || !aligned4(w_scale) || !aligned16(xq) || !aligned4(a_scale) ||
            !aligned4(y))
            return PF_EINVAL;
        const size_t yb = (size_t)N * 4;
        if (overlap(y, yb, W, (size_t)N * K) || overlap(y, yb, w_scale, yb) ||
            overlap(y, yb, xq, (size_t)K) || overlap(y, yb, a_scale, 4))
            return PF_EINVAL;
        if (pf_status st = check_device()) return st;
        GemmSet set;
        std::memset(&set, 0, sizeof(set));
        set.nprob = 1;
        char* none = nullptr;
        make_skinny(set.p[0], W, w_scale, N, K, xq, K, a_scale, 1, y, N, unsplit(N, K), none, 1);
        finish_set(set, 0);
        return launched(launch_gemv(set, (hipStream_t)stream));
    } catch (...) {
        return PF_EINTERNAL;
    }
}

size_t pf_prefill_stack_workspace(const pf_stack* stack, int64_t chunk)
{
    if (!stack || stack->n_layers <= 0 || stack->hidden <= 0 || stack->ffn <= 0 || chunk <= 0) return 0;
    // A call runs chunks of min(chunk, P) tokens.  The layout grows with the
    // chunk inside each of its two regimes (up to 64 tokens: more slots and
    // split partials; above: fewer slots), so the largest of the two regime
    // tops covers every prompt length.
    const int64_t L = stack->n_layers, H = stack->hidden, F = stack->ffn;
    const bool attn = stack->n_heads > 0;
    return std::max(stack_layout(L, H, F, chunk, attn).total,
                    stack_layout(L, H, F, std::min<int64_t>(chunk, 64), attn).total);
}

pf_status pf_prefill_stack(const pf_stack* stack, const float* x, int64_t P, int64_t chunk,
                           float* y, float* proj, float* kv, void* workspace, size_t ws_bytes,
                           pf_stack_stats* stats, void* stream)
{
    try {
        if (pf_status st = validate_stack(stack)) return st;
        if (P < 0 || chunk <= 0 || chunk > INT32_MAX || P > INT32_MAX) return PF_EINVAL;
        const int64_t L = stack->n_layers, H = stack->hidden, F = stack->ffn;
        const int64_t NT = 5 * H + 2 * F;
        const bool timed = stats && stats->time_kernels;
        if (P == 0) {
            if (stats) {
                const int max_groups = stats->max_groups;
                std::memset(stats, 0, sizeof(*stats));
                stats->time_kernels = timed ? 1 : 0;
                stats->max_groups = max_groups;
            }
            return PF_OK;
        }
        if (!x || !y || !aligned16(x) || !aligned4(y) || (proj && !aligned16(proj)))
            return PF_EINVAL;
        const size_t xb = (size_t)P * H * 4, pb = proj ? (size_t)L * P * NT * 4 : 0;
        if (overlap(x, xb, y, xb) || overlap(proj, pb, x, xb) || overlap(proj, pb, y, xb))
            return PF_EINVAL;
        const bool attn = stack->n_heads > 0;
        const size_t kb = attn ? (size_t)L * 2 * P * H * 4 : 0;
        if (attn && (!kv || !aligned16(kv) || overlap(kv, kb, x, xb) || overlap(kv, kb, y, xb) ||
                     overlap(kv, kb, proj, pb)))
            return PF_EINVAL;
        const int64_t ch = std::min(chunk, P);
        if ((uint64_t)ch * (uint64_t)std::max(H, F) >= (1ull << 32)) return PF_EINVAL;   // 32-bit offsets
        const StackLayout lay = stack_layout(L, H, F, ch, attn);
        if (!workspace || ws_bytes < lay.total) return PF_EWORKSPACE;
        if (!aligned16(workspace)) return PF_EINVAL;
        if (overlap(workspace, ws_bytes, x, xb) || overlap(workspace, ws_bytes, y, xb) ||
            overlap(workspace, ws_bytes, proj, pb) || overlap(workspace, ws_bytes, kv, kb))
            return PF_EINVAL;
        if (pf_status st = check_device()) return st;
        StackRun run{stack, x, P, ch, y, proj, attn ? kv : nullptr, static_cast<char*>(workspace), lay,
                     (hipStream_t)stream};
        Recorder rec(run.s, stats != nullptr, timed);
        const bool per_token = per_token_mode();
        // chunk groups on library streams when there are chunks for more than one
        DevStreams* ds = dev_streams();
        const int64_t C = (P + ch - 1) / ch;
        std::unique_lock<std::mutex> lock;
        if (!per_token && ds && C >= 2 && lay.groups >= 2) {
            lock = std::unique_lock<std::mutex>(ds->mu);
            if (ensure_streams(ds) == PF_OK) run.ng = (int)std::min<int64_t>(lay.groups, C);
            if (stats && stats->max_groups > 0) run.ng = std::min(run.ng, stats->max_groups);
        }
        run.ds = ds;
        pf_status st = rec.begin();
        if (st == PF_OK) st = per_token ? run.per_token(rec) : run.sweep(rec);
        if (st == PF_OK) st = rec.end();
        if (st == PF_OK && stats) {
            const int max_groups = stats->max_groups;
            std::memset(stats, 0, sizeof(*stats));
            stats->time_kernels = timed ? 1 : 0;
            stats->max_groups = max_groups;
            stats->groups = run.ng;
            stats->per_token_mode = per_token ? 1 : 0;
            stats->chunks = per_token ? P : (P + ch - 1) / ch;
            stats->tail_tokens = per_token ? 1 : P - (stats->chunks - 1) * ch;
            rec.fill(stats);
        }
        return st;
    } catch (...) {
        return PF_EINTERNAL;
    }
}

size_t pf_prefill_stack_streamed_workspace(const pf_stack* stack, int64_t P, int64_t n_buffers)
{
    if (!stack || stack->hidden <= 0 || stack->ffn <= 0 || P <= 0 || n_buffers < 2) return 0;
    return stream_layout(stack->hidden, stack->ffn, P, n_buffers).total;
}

pf_status pf_prefill_stack_streamed(const pf_stack* stack, const float* x, int64_t P, int64_t chunk,
                                    float* y, int64_t n_buffers, void* workspace, size_t ws_bytes,
                                    pf_stream_stats* stats, void* stream)
{
    try {
        if (!stack || !stack->layers || stack->n_layers <= 0 || stack->layers_alt || stack->n_heads != 0)
            return PF_EINVAL;
        if (!valid_k(stack->hidden) || !valid_k(stack->ffn)) return PF_EINVAL;
        if (stack->activation != PF_ACT_NONE && stack->activation != PF_ACT_SWIGLU) return PF_EINVAL;
        for (int64_t l = 0; l < stack->n_layers; ++l)
            for (int j = 0; j < PF_NPROJ; ++j)
                if (!stack->layers[l].W[j] || !stack->layers[l].w_scale[j]) return PF_EINVAL;
        if (P < 0 || chunk <= 0 || chunk > INT32_MAX || P > INT32_MAX || n_buffers < 2 || n_buffers > 64)
            return PF_EINVAL;
        if (stats) {
            std::memset(stats, 0, sizeof(*stats));
            stats->n_buffers = n_buffers;
        }
        if (P == 0) return PF_OK;
        const int64_t H = stack->hidden, F = stack->ffn;
        if (!x || !y || !aligned16(x) || !aligned4(y)) return PF_EINVAL;
        const size_t xb = (size_t)P * H * 4;
        if (overlap(x, xb, y, xb)) return PF_EINVAL;
        const StreamLayout lay = stream_layout(H, F, P, n_buffers);
        if (!workspace || ws_bytes < lay.total) return PF_EWORKSPACE;
        if (!aligned16(workspace) || overlap(workspace, ws_bytes, x, xb) || overlap(workspace, ws_bytes, y, xb))
            return PF_EINVAL;
        if (pf_status st = check_device()) return st;
        DevStreams* ds = dev_streams();
        if (!ds) return PF_ENODEV;
        std::unique_lock<std::mutex> lock(ds->mu);
        if (!ds->copy && hipStreamCreateWithFlags(&ds->copy, hipStreamNonBlocking) != hipSuccess)
            return PF_ELAUNCH;
        StreamRun run{stack, x, P, std::min(chunk, P), n_buffers, y, static_cast<char*>(workspace), lay,
                      (hipStream_t)stream, ds->copy, {}, {}};
        hipEvent_t t0 = nullptr, t1 = nullptr;
        if (stats && (hipEventCreate(&t0) != hipSuccess || hipEventCreate(&t1) != hipSuccess ||
                      hipEventRecord(t0, run.s) != hipSuccess))
            return PF_ELAUNCH;
        pf_status st = run.run();
        if (st == PF_OK && stats) {
            // a layer's copy is a hit when it was complete before the compute of
            // the layer before it ended (the compute never waited on it); the
            // first layer's copy has nothing to hide behind and counts as a miss
            if (hipEventRecord(t1, run.s) != hipSuccess || hipEventSynchronize(t1) != hipSuccess) {
                st = PF_ELAUNCH;
            } else {
                float ms = 0.0f;
                (void)hipEventElapsedTime(&ms, t0, t1);
                stats->elapsed_ms = ms;
                stats->layers_copied = stack->n_layers;
                for (int64_t l = 0; l < stack->n_layers; ++l) {
                    bool hit = false;
                    if (l > 0 && hipEventElapsedTime(&ms, run.computed[l - 1], run.copied[l]) == hipSuccess)
                        hit = ms <= 0.0f;
                    if (hit) ++stats->prefetch_hits;
                    else ++stats->prefetch_misses;
                }
                const int64_t rws = 5 * H + 2 * F;
                stats->bytes_copied = (double)stack->n_layers * ((double)(4 * H + 2 * F) * H + (double)H * F + 4.0 * rws);
            }
        }
        if (t0) (void)hipEventDestroy(t0);
        if (t1) (void)hipEventDestroy(t1);
        return st;
    } catch (...) {
        return PF_EINTERNAL;
    }
}

size_t pf_moe_chunk_workspace(const pf_moe* moe, int64_t T)
{
    if (validate_moe(moe) != PF_OK || T <= 0) return 0;
    return moe_layout(moe, T).total;
}

pf_status pf_moe_chunk(const pf_moe* moe, const float* x, int64_t T, int32_t* ids,
                       float* weights, float* out, void* workspace, size_t ws_bytes,
                       void* stream)
{
    try {
        if (pf_status st = validate_moe(moe)) return st;
        if (T < 0 || T * moe->top_k > 65536) return PF_EINVAL;
        if (T == 0) return PF_OK;
        const int64_t E = moe->n_experts, k = moe->top_k, H = moe->hidden, I = moe->inter;
        if (T > 16384) return PF_EINVAL;                   // a grouping workgroup's bitmap in LDS
        if (!x || !ids || !weights || !out) return PF_EINVAL;
        if (!aligned16(x) || !aligned4(ids) || !aligned4(weights) || !aligned4(out))
            return PF_EINVAL;
        const size_t xb = (size_t)T * H * 4, ib = (size_t)T * k * 4;
        if (overlap(x, xb, out, xb) || overlap(ids, ib, weights, ib) || overlap(ids, ib, out, xb) ||
            overlap(weights, ib, out, xb) || overlap(x, xb, ids, ib) || overlap(x, xb, weights, ib))
            return PF_EINVAL;
        const MoeLayout lay = moe_layout(moe, T);
        if (!workspace || ws_bytes < lay.total) return PF_EWORKSPACE;
        if (!aligned16(workspace)) return PF_EINVAL;
        if (overlap(workspace, ws_bytes, x, xb) || overlap(workspace, ws_bytes, out, xb) ||
            overlap(workspace, ws_bytes, ids, ib) || overlap(workspace, ws_bytes, weights, ib))
            return PF_EINVAL;
        if (pf_status st = check_device()) return st;
        hipStream_t s = (hipStream_t)stream;
        char* ws = static_cast<char*>(workspace);
        int8_t* xq = reinterpret_cast<int8_t*>(ws + lay.xq);
        float* xs = reinterpret_cast<float*>(ws + lay.xs);
        float* logits = reinterpret_cast<float*>(ws + lay.logits);
        int* off = reinterpret_cast<int*>(ws + lay.off);
        int* pair_tok = reinterpret_cast<int*>(ws + lay.pair_tok);
        int* comb_row = reinterpret_cast<int*>(ws + lay.comb_row);
        float* comb_w = reinterpret_cast<float*>(ws + lay.comb_w);
        float* r = reinterpret_cast<float*>(ws + lay.r);
        int8_t* hq = reinterpret_cast<int8_t*>(ws + lay.hq);
        float* hs = reinterpret_cast<float*>(ws + lay.hs);
        float* ypair = reinterpret_cast<float*>(ws + lay.ypair);
        const int Ti = (int)T, Ei = (int)E, ki = (int)k;

        // the router launch also quantises x (its workgroups stage every token row)
        pf_status st = launched(launch_router(moe->W_router, x, Ei, (int)H, Ti, logits, xq, xs, s));
        if (!st) st = launched(launch_softmax_topk(logits, Ei, Ti, ki, (int)moe->renormalize, ids,
                                                   weights, s));
        if (!st) st = launched(launch_group(ids, weights, Ti, ki, Ei, off, pair_tok, comb_row, comb_w, s));
        if (st) return st;
        ExpertArgs gu;
        std::memset(&gu, 0, sizeof(gu));
        gu.W0 = moe->W_gate; gu.W1 = moe->W_up; gu.s0 = moe->s_gate; gu.s1 = moe->s_up;
        gu.off = off; gu.gather = pair_tok; gu.X = xq; gu.xs = xs; gu.Y = r;
        gu.ldx = H; gu.ldy = I; gu.N = (int)I; gu.K = (int)H; gu.E = Ei;
        gu.tiles_n = (int)((I + 63) / 64);
        gu.act = (int)moe->activation;
        ExpertArgs dn;
        std::memset(&dn, 0, sizeof(dn));
        dn.W0 = moe->W_down; dn.s0 = moe->s_down;
        dn.off = off; dn.gather = nullptr; dn.X = hq; dn.xs = hs; dn.Y = ypair;
        dn.ldx = I; dn.ldy = H; dn.N = (int)H; dn.K = (int)I; dn.E = Ei;
        dn.tiles_n = (int)((H + 63) / 64);
        if (moe_fused_mode() && expert_fused_shape(H, I)) {
            // gate/up, quantise(r) and down in one launch, one workgroup per expert
            st = launched(launch_expert_fused(gu, dn, s));
        } else {
            st = launched(launch_expert(gu, s));
            if (!st) st = launched(launch_quantize(r, I, Ti * ki, (int)I, hq, hs, s));
            if (!st) st = launched(launch_expert(dn, s));
        }
        if (!st) st = launched(launch_combine(ypair, comb_row, comb_w, Ti, ki, (int)H, out, s));
        return st;
    } catch (...) {
        return PF_EINTERNAL;
    }
}

pf_status pf_expf_cr(const float* x, int64_t n, float* y, void* stream)
{
    try {
        if (n < 0) return PF_EINVAL;
        if (n == 0) return PF_OK;
        if (!x || !y || !aligned4(x) || !aligned4(y)) return PF_EINVAL;
        if (overlap(x, (size_t)n * 4, y, (size_t)n * 4) && x != y) return PF_EINVAL;
        if (pf_status st = check_device()) return st;
        return launched(launch_expf(x, n, y, (hipStream_t)stream));
    } catch (...) {
        return PF_EINTERNAL;
    }
}

}  // extern "C"
