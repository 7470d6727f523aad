// moe.hip — expert prefill of one chunk on the device ("Red Lite dev24",
// What changed: route every token of the chunk, take the union of the selected
// experts, run each expert once over its token group).
//
// Router -> softmax/top-k -> grouping -> gate/up product (with r = g * u fused in
// the epilogue) -> per-row quantisation -> down product -> weighted combine.
// No host round trip: the expert plan stays in device memory.
#include "device.hpp"
#include "kernels.hpp"
#include "expf_cr.hpp"
#include "lds_dma.hpp"

namespace pf {

// ---------------------------------------------------------------------------
// Router logits: l[t][e] = sum over k ascending of fl(Wr[e][k] * x[t][k]), each
// product and each partial sum rounded on its own (no fused multiply-add: the
// library is compiled with -ffp-contract=off).  32 tokens x 32 experts per
// workgroup; a thread owns TI tokens x EJ experts, each an independent chain;
// 64-wide k pieces staged in LDS, double-buffered: the next piece is loaded
// into registers while the current one is consumed.
constexpr int kRtTile = 32;
constexpr int kRtK = 64;
constexpr int kRtTI = 1, kRtEJ = 2;                    // chains per thread: tokens x experts

// With xq non-null the launch also quantises x per token (a1's definition): a
// workgroup stages all H values of its 32 tokens anyway, so it keeps their exact
// absolute maxima on the way; workgroup (bx, by) then writes the codes and
// scales of its share of the 32 rows, re-reading them from L2.
template <int TI, int EJ>
__global__ __launch_bounds__(1024 / (TI * EJ)) void k_router(const float* __restrict__ Wr,
                                                             const float* __restrict__ x, int E, int H, int T,
                                                             float* __restrict__ logits,
                                                             int8_t* __restrict__ xq,
                                                             float* __restrict__ xs)
{
    constexpr int NT = 1024 / (TI * EJ);                // threads
    constexpr int CE = kRtTile / EJ, CT = kRtTile / TI;  // thread grid: CE experts x CT tokens
    constexpr int NP = kRtTile * kRtK / 4;              // float4 pieces per operand and piece
    constexpr int NF = (NP + NT - 1) / NT;              // of them per thread
    static_assert(NP % NT == 0 || NT % NP == 0, "staging split");
    const bool stager = (int)threadIdx.x < NP;          // false only with more threads than pieces
    // rows padded to 68 floats: 16-byte aligned, and the 16 rows a quarter-wave
    // reads at one k sit in distinct banks
    __shared__ __attribute__((aligned(16))) float sx[2][kRtTile][kRtK + 4];
    __shared__ __attribute__((aligned(16))) float sw[2][kRtTile][kRtK + 4];
    const int e0 = blockIdx.x * kRtTile, t0 = blockIdx.y * kRtTile;
    const int ei = threadIdx.x % CE, ti = threadIdx.x / CE;
    // staging: float4 f = threadIdx.x + NT u of a [32][64] piece -> row f / 16,
    // column 4 (f % 16); rows past the end repeat the last one
    int rr[NF], cc[NF];
    const float* xr[NF];
    const float* wr[NF];
    float4 px[NF], pw[NF];
    float am[NF];                                       // running |x| maxima of the staged rows
#pragma unroll
    for (int u = 0; u < NF; ++u) {
        const int f = ((int)threadIdx.x + NT * u) % NP;
        rr[u] = f >> 4;
        cc[u] = (f & 15) << 2;
        xr[u] = x + (int64_t)min(t0 + rr[u], T - 1) * H + cc[u];
        wr[u] = Wr + (int64_t)min(e0 + rr[u], E - 1) * H + cc[u];
        px[u] = *reinterpret_cast<const float4*>(xr[u]);
        pw[u] = *reinterpret_cast<const float4*>(wr[u]);
        am[u] = fmaxf(fmaxf(fabsf(px[u].x), fabsf(px[u].y)), fmaxf(fabsf(px[u].z), fabsf(px[u].w)));
    }
    if (stager) {
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            *reinterpret_cast<float4*>(&sx[0][rr[u]][cc[u]]) = px[u];
            *reinterpret_cast<float4*>(&sw[0][rr[u]][cc[u]]) = pw[u];
        }
    }
    float acc[TI][EJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < EJ; ++j) acc[i][j] = 0.0f;
    const int npieces = H / kRtK;
    __syncthreads();
    for (int pc = 0; pc < npieces; ++pc) {
        const int b = pc & 1;
        const bool more = pc + 1 < npieces;
        if (more && stager) {
            const int k1 = (pc + 1) * kRtK;
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                px[u] = *reinterpret_cast<const float4*>(xr[u] + k1);
                pw[u] = *reinterpret_cast<const float4*>(wr[u] + k1);
            }
        }
#pragma unroll 4
        for (int kk = 0; kk < kRtK; kk += 4) {
            float4 wv[EJ], xv[TI];
#pragma unroll
            for (int j = 0; j < EJ; ++j) wv[j] = *reinterpret_cast<const float4*>(&sw[b][ei + CE * j][kk]);
#pragma unroll
            for (int i = 0; i < TI; ++i) xv[i] = *reinterpret_cast<const float4*>(&sx[b][ti + CT * i][kk]);
#pragma unroll
            for (int c = 0; c < 4; ++c)                  // k ascending within each chain
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int j = 0; j < EJ; ++j) acc[i][j] = acc[i][j] + wv[j][c] * xv[i][c];
        }
        if (more && stager) {
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                *reinterpret_cast<float4*>(&sx[b ^ 1][rr[u]][cc[u]]) = px[u];
                *reinterpret_cast<float4*>(&sw[b ^ 1][rr[u]][cc[u]]) = pw[u];
                am[u] = fmaxf(am[u], fmaxf(fmaxf(fabsf(px[u].x), fabsf(px[u].y)),
                                           fmaxf(fabsf(px[u].z), fabsf(px[u].w))));
            }
        }
        __syncthreads();
    }
    if (xq) {
        // the row maxima: the 16 stagers of a row are 16 consecutive lanes
        static_assert(NF == 1 && NP == NT, "one staged piece per thread and piece");
        __shared__ float samax[kRtTile];
        float m = am[0];
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        if ((threadIdx.x & 15) == 0) samax[rr[0]] = m;
        __syncthreads();
        // this workgroup's rows of the 32: an equal share per expert tile
        const int per = (kRtTile + gridDim.x - 1) / gridDim.x;
        const int r0 = blockIdx.x * per, r1 = min(r0 + per, kRtTile);
        const int n4 = H >> 2;
        for (int r = r0; r < r1 && t0 + r < T; ++r) {
            const float sc = samax[r] / 127.0f;
            if (threadIdx.x == 0) xs[t0 + r] = sc;
            const float4* row = reinterpret_cast<const float4*>(x + (int64_t)(t0 + r) * H);
            int* qrow = reinterpret_cast<int*>(xq + (int64_t)(t0 + r) * H);
            for (int i = threadIdx.x; i < n4; i += NT) {
                int packed = 0;
                if (sc != 0.0f) {
                    const float4 v = row[i];
                    packed = (quant_code(v.x, sc) & 0xff) | ((quant_code(v.y, sc) & 0xff) << 8) |
                             ((quant_code(v.z, sc) & 0xff) << 16) | ((quant_code(v.w, sc) & 0xff) << 24);
                }
                qrow[i] = packed;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < EJ; ++j) {
            const int t = t0 + ti + CT * i, e = e0 + ei + CE * j;
            if (t < T && e < E) logits[(int64_t)t * E + e] = acc[i][j];
        }
}

hipError_t launch_router(const float* Wr, const float* x, int E, int H, int T, float* logits,
                         int8_t* xq, float* xs, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    dim3 g((E + kRtTile - 1) / kRtTile, (T + kRtTile - 1) / kRtTile);
    PF_LAUNCH((k_router<kRtTI, kRtEJ>), g, dim3(1024 / (kRtTI * kRtEJ)), 0, s, Wr, x, E, H, T, logits, xq, xs);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_expf(const float* __restrict__ x, int64_t n,
                                              float* __restrict__ y)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        y[i] = expf_cr(x[i]);
}

hipError_t launch_expf(const float* x, int64_t n, float* y, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    PF_LAUNCH(k_expf, dim3((unsigned)blocks), dim3(256), 0, s, x, n, y);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Softmax and top-k, one workgroup per token, one thread per expert.
// m = max l (exact, any order); z_e = expf_cr(l_e - m); S = z_0 + z_1 + ... in
// ascending e (one lane, sequential, over LDS); p_e = z_e / S.  Each wave then
// takes the k best keys (p, -e) of its 64 experts by k rounds of a wave-wide
// maximum; wave 0 takes the k best of those candidates the same way, so ties
// go to the lower expert id.
constexpr int kSmMaxE = 1024;
constexpr int kSmMaxK = 32;

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(v, off);
        v = o > v ? o : v;
    }
    return v;
}

__global__ __launch_bounds__(1024) void k_softmax_topk(const float* __restrict__ logits, int E, int T,
                                                       int k, int renorm, int* __restrict__ ids,
                                                       float* __restrict__ w)
{
    __shared__ __attribute__((aligned(16))) float zs[kSmMaxE];
    __shared__ float wmax[kSmMaxE / 64];
    __shared__ float sS;
    __shared__ unsigned long long cand[kSmMaxE / 64 * kSmMaxK];
    const int t = blockIdx.x;
    const int e = threadIdx.x, lane = e & 63, wave = e >> 6, nw = blockDim.x >> 6;
    const float* row = logits + (int64_t)t * E;
    const float l = e < E ? row[e] : -__builtin_huge_valf();
    float m = wave_max(l);
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
    m = wmax[0];
    for (int i = 1; i < nw; ++i) m = fmaxf(m, wmax[i]);
    const float z = e < E ? expf_cr(l - m) : 0.0f;
    zs[e] = z;                                           // zeros past E add nothing below
    __syncthreads();
    if (e == 0) {
        float S = 0.0f;
        for (int i = 0; i < (int)blockDim.x; i += 4) {
            const float4 q = *reinterpret_cast<const float4*>(zs + i);
            S = S + q.x;
            S = S + q.y;
            S = S + q.z;
            S = S + q.w;
        }
        sS = S;
    }
    __syncthreads();
    const float p = z / sS;
    const int kw = min(k, 64);                           // candidates per wave
    unsigned long long key =
        e < E ? ((unsigned long long)__float_as_uint(p) << 32) | (unsigned long long)(0xffffffffu - (unsigned)e) : 0ull;
    for (int j = 0; j < kw; ++j) {
        const unsigned long long best = wave_max_u64(key);
        if (key == best) key = 0ull;                     // keys are distinct (distinct e)
        if (lane == 0) cand[wave * kw + j] = best;
    }
    __syncthreads();
    // the k best of the nw * kw candidates: candidate i's place is the number of
    // candidates above it (the keys are distinct), so every candidate finds its
    // place at once and the first k write their (id, weight)
    const int nc = nw * kw;
    __shared__ float chosen[kSmMaxK];
    int place = k;
    unsigned long long mine = 0ull;
    if (e < nc) {
        mine = cand[e];
        place = 0;
        for (int j = 0; j < nc; ++j) place += cand[j] > mine;
        if (place < k) {
            ids[(int64_t)t * k + place] = (int)(0xffffffffu - (unsigned)(mine & 0xffffffffu));
            chosen[place] = __uint_as_float((unsigned)(mine >> 32));
        }
    }
    if (!renorm) {
        if (place < k) w[(int64_t)t * k + place] = chosen[place];
        return;
    }
    // renormalised over the chosen: T = the chosen p summed in rank order
    // (one lane, sequentially), then w = p / T
    __syncthreads();
    __shared__ float sT;
    if (e == 0) {
        float Tk = 0.0f;
        for (int j = 0; j < k; ++j) Tk = Tk + chosen[j];
        sT = Tk;
    }
    __syncthreads();
    if (place < k) w[(int64_t)t * k + place] = chosen[place] / sT;
}

hipError_t launch_softmax_topk(const float* logits, int E, int T, int k, int renorm, int* ids,
                               float* w, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    if (E > kSmMaxE || k > kSmMaxK) return hipErrorInvalidValue;
    PF_LAUNCH(k_softmax_topk, dim3(T), dim3(64 * ((E + 63) / 64)), 0, s, logits, E, T, k, renorm, ids, w);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouping by the union of selected experts.  Workgroup g of the grid owns
// experts [g * kGrpE, (g + 1) * kGrpE).  Every workgroup counts the pairs of
// every expert (LDS atomics) and scans the counts into the offsets (workgroup 0
// writes them), and keeps an (expert x token) selection bitmap of its own
// experts.  Then every pair of its experts independently: its row in the
// expert's group is off[e] + the number of tokens below t that chose e (a
// popcount over e's bitmap words), so each expert lists its tokens in
// ascending order; its rank among t's selections is the number of t's ids
// below e, which orders the combine table by ascending expert id.  With kLds
// the ids are first copied into LDS, so the per-pair reads do not go to memory.
constexpr int kGrpE = 16;

template <bool kLds>
__global__ __launch_bounds__(1024) void k_group(const int* __restrict__ ids_g,
                                                const float* __restrict__ w, int T, int k, int E,
                                                int* __restrict__ off, int* __restrict__ pair_tok,
                                                int* __restrict__ comb_row,
                                                float* __restrict__ comb_w)
{
    extern __shared__ unsigned sel[];                   // [kGrpE][words], then the ids (kLds)
    __shared__ int cnt[1024];
    __shared__ int scan[1024];
    __shared__ int wsum[16];
    const int words = (T + 31) >> 5;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int np = T * k;
    const int e0 = (int)blockIdx.x * kGrpE, e1 = min(e0 + kGrpE, E);
    int* ids_l = reinterpret_cast<int*>(sel + kGrpE * words);
    if (kLds) {
        for (int p0 = 0; p0 < np; p0 += 4 * 1024) {
            int v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int p = p0 + u * 1024 + tid;
                v[u] = p < np ? ids_g[p] : 0;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int p = p0 + u * 1024 + tid;
                if (p < np) ids_l[p] = v[u];
            }
        }
    }
    const int* ids = kLds ? ids_l : ids_g;
    for (int i = tid; i < kGrpE * words; i += 1024) sel[i] = 0;
    cnt[tid] = 0;
    __syncthreads();
    for (int p = tid; p < np; p += 1024) {
        const int t = p / k, e = ids[p];
        atomicAdd(&cnt[e], 1);
        if (e >= e0 && e < e1) atomicOr(&sel[(e - e0) * words + (t >> 5)], 1u << (t & 31));
    }
    __syncthreads();
    // inclusive scan of cnt[0..1024): within each wave by lane shuffles, then
    // the 16 wave totals
    int v = cnt[tid];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d);
        if (lane >= d) v += o;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    for (int i = 0; i < wave; ++i) v += wsum[i];
    scan[tid] = v;
    __syncthreads();
    if (blockIdx.x == 0) {
        if (tid < E) off[tid + 1] = scan[tid];
        if (tid == 0) off[0] = 0;
    }
    for (int p = tid; p < np; p += 1024) {
        const int e = ids[p];
        if (e < e0 || e >= e1) continue;
        const int t = p / k;
        const unsigned* se = sel + (e - e0) * words;
        int below = __popc(se[t >> 5] & ((1u << (t & 31)) - 1u));
        for (int wd = 0; wd < (t >> 5); ++wd) below += __popc(se[wd]);
        const int pos = scan[e] - cnt[e] + below;
        int rank = 0;
        for (int j = 0; j < k; ++j) rank += ids[t * k + j] < e;
        pair_tok[pos] = t;
        comb_row[t * k + rank] = pos;
        comb_w[t * k + rank] = w[p];
    }
}

hipError_t launch_group(const int* ids, const float* w, int T, int k, int E, int* off,
                        int* pair_tok, int* comb_row, float* comb_w, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    const size_t lds = group_lds_bytes(T, kGrpE), with_ids = lds + (size_t)T * k * 4;
    const dim3 g((E + kGrpE - 1) / kGrpE);
    if (with_ids <= 64 * 1024)
        PF_LAUNCH(k_group<true>, g, dim3(1024), with_ids, s, ids, w, T, k, E, off, pair_tok, comb_row, comb_w);
    else
        PF_LAUNCH(k_group<false>, g, dim3(1024), lds, s, ids, w, T, k, E, off, pair_tok, comb_row, comb_w);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Expert products.  Workgroup = (expert e, band of 64 rows); the expert's token
// group (pairs off[e] .. off[e+1]) is processed 32 tokens at a time, so a group
// of up to 32 tokens reads the expert's weight band exactly once; an unselected
// expert returns at once and reads no weight.  With two weights (gate and up)
// the epilogue writes r = fl(g * u).
constexpr int kExPiece = 8;
constexpr int kExStride = kExPiece * 64 + 16;
constexpr int kExTB = 2;

template <bool kPair>
__global__ __launch_bounds__(256) void k_expert(ExpertArgs A)
{
    __shared__ __attribute__((aligned(16))) int8_t xl[16 * kExTB * kExStride];
    __shared__ int rows[16 * kExTB];
    const int e = blockIdx.x / A.tiles_n, tn = blockIdx.x % A.tiles_n;
    const int p0 = A.off[e], p1 = A.off[e + 1];
    if (p0 == p1) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw0 = tn * 64 + wave * 16;
    const int nkb = A.K >> 6;
    const int arow = min(nw0 + (lane & 15), A.N - 1);
    const int64_t wbase = (int64_t)e * A.N * A.K + (int64_t)arow * A.K + ((lane >> 4) << 4);
    const int8_t* w0 = A.W0 + wbase;
    const int8_t* w1 = kPair ? A.W1 + wbase : nullptr;
    const int boff = (lane & 15) * kExStride + ((lane >> 4) << 4);
    const int nr = nw0 + ((lane >> 4) << 2);

    for (int g0 = p0; g0 < p1; g0 += 16 * kExTB) {
        const int gm = min(16 * kExTB, p1 - g0);
        __syncthreads();
        if (threadIdx.x < 16 * kExTB)
            rows[threadIdx.x] = threadIdx.x < gm
                                    ? (A.gather ? A.gather[g0 + threadIdx.x] : g0 + threadIdx.x)
                                    : -1;
        v4i acc0[kExTB], acc1[kExTB];
#pragma unroll
        for (int tb = 0; tb < kExTB; ++tb) acc0[tb] = acc1[tb] = v4i{0, 0, 0, 0};
        for (int kp = 0; kp < nkb; kp += kExPiece) {
            const int npc = min(kExPiece, nkb - kp);
            v4i a0[kExPiece], a1[kExPiece];
#pragma unroll
            for (int i = 0; i < kExPiece; ++i)
                if (i < npc) {
                    a0[i] = ld16(w0 + (int64_t)(kp + i) * 64);
                    if (kPair) a1[i] = ld16(w1 + (int64_t)(kp + i) * 64);
                }
            __syncthreads();
            const int cpr = npc * 4;
            for (int idx = threadIdx.x; idx < 16 * kExTB * cpr; idx += 256) {
                const int t = idx / cpr, c = idx - t * cpr;
                const int r = rows[t];
                v4i v = v4i{0, 0, 0, 0};
                if (r >= 0) v = ld16(A.X + (int64_t)r * A.ldx + (int64_t)kp * 64 + c * 16);
                st16(xl + t * kExStride + c * 16, v);
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kExPiece; ++i) {
                if (i < npc) {
#pragma unroll
                    for (int tb = 0; tb < kExTB; ++tb) {
                        const v4i b = *reinterpret_cast<const v4i*>(xl + tb * 16 * kExStride + boff + i * 64);
                        acc0[tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[i], b, acc0[tb], 0, 0, 0);
                        if (kPair)
                            acc1[tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[i], b, acc1[tb], 0, 0, 0);
                    }
                }
            }
        }
#pragma unroll
        for (int tb = 0; tb < kExTB; ++tb) {
            const int j = tb * 16 + (lane & 15);
            if (j >= gm) continue;
            const int r = rows[j];
            const float xs = A.xs[r];
            float* yrow = A.Y + (int64_t)(g0 + j) * A.ldy;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = nr + q;
                if (n >= A.N) continue;
                const float g = epilogue(acc0[tb][q], A.s0[(int64_t)e * A.N + n], xs);
                if (kPair) {
                    const float u = epilogue(acc1[tb][q], A.s1[(int64_t)e * A.N + n], xs);
                    yrow[n] = (A.act ? silu_cr(g) : g) * u;
                } else {
                    yrow[n] = g;
                }
            }
        }
    }
}

// Streaming form for K = 64 KB.  Workgroup = (expert e, band of 64 RB weight
// rows; with two weights, 64 rows of each).  Per token group of up to 32:
// the group's token rows are copied once into LDS, as 1 KB fragments (token
// block tb, k-block kb) laid out as the MFMA B operand wants them.  Each wave
// then streams its weight rows straight into registers: RB row blocks of 16
// rows one after the other, each over all KB k-blocks, D fragments (16 rows x
// 64 bytes of each weight) ahead across row-block boundaries, with no barrier
// inside the stream.  The stream is unrolled, so every ring slot and wait is
// fixed at compile time.
template <bool kPair, int RB, int D, int KB, bool kSilu = false>
__global__ __launch_bounds__(256) void k_expert_stream(ExpertArgs A)
{
    constexpr int M = kPair ? 2 : 1;              // weights read per fragment
    constexpr int NF = RB * KB;                   // fragments per wave
    static_assert(D <= NF, "ring within the stream");
    __shared__ __attribute__((aligned(16))) int8_t xl[2 * KB * 1024];
    __shared__ int rows[32];
    const int e = blockIdx.x / A.tiles_n, tn = blockIdx.x % A.tiles_n;
    const int p0 = A.off[e], p1 = A.off[e + 1];
    if (p0 == p1) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int koff = (lane >> 4) << 4;
    const int r0 = tn * 64 * RB + wave * 16 * RB; // this wave's first weight row
    // weight pointers of row block 0 (row clamped into the matrix; rows past
    // N are never stored); row block rb is rb * 16 rows further
    const int8_t* wp[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        wp[m] = (kPair && m == 1 ? A.W1 : A.W0) + (int64_t)e * A.N * A.K + koff;
    auto frag = [&](int m, int f) {               // fragment f = (rb, kb) of weight m
        const int rb = f / KB, kb = f % KB;
        const int row = min(r0 + rb * 16 + (lane & 15), A.N - 1);
        return ld16(wp[m] + (int64_t)row * A.K + kb * 64);
    };

    for (int g0 = p0; g0 < p1; g0 += 32) {
        const int gm = min(32, p1 - g0);
        __syncthreads();                           // the previous group's LDS reads are done
        if (threadIdx.x < 32)
            rows[threadIdx.x] = (int)threadIdx.x < gm
                                    ? (A.gather ? A.gather[g0 + threadIdx.x] : g0 + threadIdx.x)
                                    : -1;
        __syncthreads();
        // the epilogues' scales, loaded before the stream (a load issued inside
        // it would be waited for together with every weight load before it)
        float xsv[2], ws0[RB][4], ws1[RB][4];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int j = tb * 16 + (lane & 15);
            xsv[tb] = A.xs[rows[j] >= 0 ? rows[j] : rows[0]];
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = min(r0 + rb * 16 + ((lane >> 4) << 2) + q, A.N - 1);
                ws0[rb][q] = A.s0[(int64_t)e * A.N + n];
                if (kPair) ws1[rb][q] = A.s1[(int64_t)e * A.N + n];
            }
        // token fragments: (tb, kb) at (tb * KB + kb) KB; lane l brings token
        // (l & 15) of the block, bytes (l >> 4) * 16 .. + 15 of the k-block;
        // wave w brings fragments w, w + 4, ...  Token slots past the group
        // read row rows[0] and are never stored.  Loaded into registers first,
        // then the first D weight fragments are issued, so both are in flight
        // together.
        v4i xv[2 * KB / 4];
        {
            const int rl = rows[lane & 15], rh = rows[16 + (lane & 15)];
            const int8_t* x0 = A.X + (int64_t)(rl >= 0 ? rl : rows[0]) * A.ldx + koff;
            const int8_t* x1 = A.X + (int64_t)(rh >= 0 ? rh : rows[0]) * A.ldx + koff;
#pragma unroll
            for (int i = 0; i < 2 * KB / 4; ++i) {
                const int f = wave + 4 * i;
                xv[i] = ld16(f < KB ? x0 + (int64_t)f * 64 : x1 + (int64_t)(f - KB) * 64);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        v4i ring[D][M];
#pragma unroll
        for (int f = 0; f < D; ++f)
#pragma unroll
            for (int m = 0; m < M; ++m) ring[f][m] = frag(m, f);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 2 * KB / 4; ++i) st16(xl + (wave + 4 * i) * 1024 + lane * 16, xv[i]);
        // the LDS writes are complete (lgkmcnt 0; the loads stay in flight),
        // then every wave's are visible after the barrier
        __builtin_amdgcn_s_waitcnt(0xC07F);
        stage_barrier();

        v4i acc[M][2];
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int rb = f / KB, kb = f % KB;
            if (kb == 0) {
#pragma unroll
                for (int m = 0; m < M; ++m) acc[m][0] = acc[m][1] = v4i{0, 0, 0, 0};
            }
            const v4i b0 = *reinterpret_cast<const v4i*>(xl + kb * 1024 + lane * 16);
            const v4i b1 = *reinterpret_cast<const v4i*>(xl + (KB + kb) * 1024 + lane * 16);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                acc[m][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ring[f % D][m], b0, acc[m][0], 0, 0, 0);
                acc[m][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ring[f % D][m], b1, acc[m][1], 0, 0, 0);
            }
            if (f + D < NF) {
#pragma unroll
                for (int m = 0; m < M; ++m) ring[f % D][m] = frag(m, f + D);
            }
            __builtin_amdgcn_sched_barrier(0);     // keep each refill D fragments ahead of its use
            if (kb == KB - 1) {
                // epilogue of row block rb: acc[m][tb][q] is weight row
                // r0 + rb * 16 + (lane >> 4) * 4 + q, token tb * 16 + (lane & 15)
                const int nr = r0 + rb * 16 + ((lane >> 4) << 2);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    const int j = tb * 16 + (lane & 15);
                    if (j >= gm) continue;
                    float* yrow = A.Y + (int64_t)(g0 + j) * A.ldy;
                    float4 v;
                    float* vp = &v.x;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float g = epilogue(acc[0][tb][q], ws0[rb][q], xsv[tb]);
                        if (kPair) {
                            const float u = epilogue(acc[M - 1][tb][q], ws1[rb][q], xsv[tb]);
                            vp[q] = (kSilu ? silu_cr(g) : g) * u;
                        } else {
                            vp[q] = g;
                        }
                    }
                    if (nr + 3 < A.N) {
                        *reinterpret_cast<float4*>(yrow + nr) = v;
                    } else {
#pragma unroll
                        for (int q = 0; q < 3; ++q)
                            if (nr + q < A.N) yrow[nr + q] = vp[q];
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The whole expert pipeline in one workgroup per expert ("Red Lite dev24",
// Scope boundary: the gate/up/down expert kernel).  Over each group of up to
// 32 of the expert's (token, expert) pairs: gate/up over every 64-row band
// (r = fl(g u), or fl(silu(g) u), to the pairs' rows of G.Y, and each row's
// |r| maximum into LDS by integer atomics on its binary32 bits, exact for
// non-negative values); then the rows' codes, quantise(r) per pair row with
// the same arithmetic as k_quantize_rows, written straight into LDS as the
// down product's B fragments; then down over every band of 64 RBD rows to the
// pairs' rows of Dn.Y.  r is read back by the workgroup that wrote it, and
// neither the quantisation nor down waits for another launch.  Each wave
// streams its weight rows into registers D fragments ahead, across band
// boundaries, as k_expert_stream does within one band.
template <int KBG, int KBD, bool kSilu>
__global__ __launch_bounds__(256) void k_expert_fused(ExpertArgs G, ExpertArgs Dn)
{
    constexpr int DG = 8, DD = 16;                // fragments ahead: gate/up, down
    constexpr int RBD = KBD == 32 ? 2 : 4;        // down row blocks of 16 per wave and band
    constexpr int NFG = KBG, NFD = RBD * KBD;     // fragments per wave and band
    static_assert(NFG % DG == 0 && NFD % DD == 0, "ring slots the same in every band");
    constexpr int KX = KBG > KBD ? KBG : KBD;
    __shared__ __attribute__((aligned(16))) int8_t xl[2 * KX * 1024];
    __shared__ int rows[32];
    __shared__ unsigned int rmax[32];
    __shared__ float rsc[32];
    const int e = blockIdx.x;
    const int p0 = G.off[e], p1 = G.off[e + 1];
    if (p0 == p1) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int koff = (lane >> 4) << 4;
    const int I = G.N, H = Dn.N;                  // gate/up rows (K = H); down rows (K = I)
    const int tiles_g = (I + 63) / 64, tiles_d = (H + 64 * RBD - 1) / (64 * RBD);
    const int8_t* wg = G.W0 + (int64_t)e * I * H + koff;
    const int8_t* wu = G.W1 + (int64_t)e * I * H + koff;
    const int8_t* wd = Dn.W0 + (int64_t)e * H * I + koff;
    auto gfrag = [&](const int8_t* w, int tn, int kb) {   // band tn, k-block kb (16 rows per wave)
        const int row = min(tn * 64 + wave * 16 + (lane & 15), I - 1);
        return ld16(w + (int64_t)row * H + kb * 64);
    };
    auto dfrag = [&](int tn, int f) {                    // band tn, fragment (rb, kb)
        const int rb = f / KBD, kb = f % KBD;
        const int row = min(tn * 64 * RBD + wave * 16 * RBD + rb * 16 + (lane & 15), H - 1);
        return ld16(wd + (int64_t)row * I + kb * 64);
    };

    for (int g0 = p0; g0 < p1; g0 += 32) {
        const int gm = min(32, p1 - g0);
        __syncthreads();                           // the previous group's LDS reads are done
        if (threadIdx.x < 32) {
            rows[threadIdx.x] = (int)threadIdx.x < gm ? G.gather[g0 + threadIdx.x] : -1;
            rmax[threadIdx.x] = 0u;
        }
        __syncthreads();
        float xsv[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int j = tb * 16 + (lane & 15);
            xsv[tb] = G.xs[rows[j] >= 0 ? rows[j] : rows[0]];
        }
        // token fragments (tb, kb) at (tb * KBG + kb) KB, loaded into registers,
        // then the first weight fragments, so both are in flight together
        v4i ring[DG][2];
        {
            v4i xv[2 * KBG / 4];
            const int rl = rows[lane & 15], rh = rows[16 + (lane & 15)];
            const int8_t* x0 = G.X + (int64_t)(rl >= 0 ? rl : rows[0]) * G.ldx + koff;
            const int8_t* x1 = G.X + (int64_t)(rh >= 0 ? rh : rows[0]) * G.ldx + koff;
#pragma unroll
            for (int i = 0; i < 2 * KBG / 4; ++i) {
                const int f = wave + 4 * i;
                xv[i] = ld16(f < KBG ? x0 + (int64_t)f * 64 : x1 + (int64_t)(f - KBG) * 64);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int f = 0; f < DG; ++f) {
                ring[f][0] = gfrag(wg, 0, f);
                ring[f][1] = gfrag(wu, 0, f);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 2 * KBG / 4; ++i) st16(xl + (wave + 4 * i) * 1024 + lane * 16, xv[i]);
            __builtin_amdgcn_s_waitcnt(0xC07F);    // LDS writes done, the loads stay in flight
            stage_barrier();
        }
        // gate/up, band by band
        for (int tn = 0; tn < tiles_g; ++tn) {
            const int nr = tn * 64 + wave * 16 + ((lane >> 4) << 2);
            float ws0[4], ws1[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = min(nr + q, I - 1);
                ws0[q] = G.s0[(int64_t)e * I + n];
                ws1[q] = G.s1[(int64_t)e * I + n];
            }
            v4i acc[2][2];
#pragma unroll
            for (int m = 0; m < 2; ++m) acc[m][0] = acc[m][1] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int f = 0; f < NFG; ++f) {
                const v4i b0 = *reinterpret_cast<const v4i*>(xl + f * 1024 + lane * 16);
                const v4i b1 = *reinterpret_cast<const v4i*>(xl + (KBG + f) * 1024 + lane * 16);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    acc[m][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ring[f % DG][m], b0, acc[m][0], 0, 0, 0);
                    acc[m][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ring[f % DG][m], b1, acc[m][1], 0, 0, 0);
                }
                if (f + DG < NFG) {
                    ring[f % DG][0] = gfrag(wg, tn, f + DG);
                    ring[f % DG][1] = gfrag(wu, tn, f + DG);
                } else if (tn + 1 < tiles_g) {             // the next band's first fragments
                    ring[f % DG][0] = gfrag(wg, tn + 1, f + DG - NFG);
                    ring[f % DG][1] = gfrag(wu, tn + 1, f + DG - NFG);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // acc[m][tb][q]: row nr + q, pair tb * 16 + (lane & 15)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const int j = tb * 16 + (lane & 15);
                float4 v;
                float* vp = &v.x;
                float m = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float g = epilogue(acc[0][tb][q], ws0[q], xsv[tb]);
                    const float u = epilogue(acc[1][tb][q], ws1[q], xsv[tb]);
                    vp[q] = (kSilu ? silu_cr(g) : g) * u;
                    if (nr + q < I) m = fmaxf(m, fabsf(vp[q]));
                }
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                if (j < gm) {
                    float* yrow = G.Y + (int64_t)(g0 + j) * G.ldy;
                    if (nr + 3 < I) {
                        *reinterpret_cast<float4*>(yrow + nr) = v;
                    } else {
#pragma unroll
                        for (int q = 0; q < 3; ++q)
                            if (nr + q < I) yrow[nr + q] = vp[q];
                    }
                    if ((lane >> 4) == 0) atomicMax(&rmax[j], __float_as_uint(m));
                }
            }
        }
        __syncthreads();                           // r in memory, the row maxima in LDS
        if (threadIdx.x < 32) rsc[threadIdx.x] = __uint_as_float(rmax[threadIdx.x]) / 127.0f;
        __syncthreads();
        // the codes: fragment (tb, kb) at (tb * KBD + kb) KB; lane l holds pair
        // tb * 16 + (l & 15), bytes (l >> 4) * 16 .. + 15 of k-block kb
#pragma unroll
        for (int i = 0; i < 2 * KBD / 4; ++i) {
            const int f = wave + 4 * i;
            const int tb = f / KBD, kb = f % KBD;
            const int j = tb * 16 + (lane & 15);
            v4i packed = v4i{0, 0, 0, 0};
            const float s = j < gm ? rsc[j] : 0.0f;
            if (s != 0.0f) {
                const float4* src =
                    reinterpret_cast<const float4*>(G.Y + (int64_t)(g0 + j) * G.ldy + kb * 64 + koff);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float4 x = src[w];
                    packed[w] = (quant_code(x.x, s) & 0xff) | ((quant_code(x.y, s) & 0xff) << 8) |
                                ((quant_code(x.z, s) & 0xff) << 16) | ((quant_code(x.w, s) & 0xff) << 24);
                }
            }
            st16(xl + f * 1024 + lane * 16, packed);
        }
        float xsd[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) xsd[tb] = rsc[tb * 16 + (lane & 15)];
        // the first down fragments travel across the barrier
        v4i dring[DD];
#pragma unroll
        for (int f = 0; f < DD; ++f) dring[f] = dfrag(0, f);
        __builtin_amdgcn_s_waitcnt(0xC07F);        // the codes are in LDS
        stage_barrier();
        // down, band by band
        for (int tn = 0; tn < tiles_d; ++tn) {
            const int r0 = tn * 64 * RBD + wave * 16 * RBD;
            float ws[RBD][4];
#pragma unroll
            for (int rb = 0; rb < RBD; ++rb)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    ws[rb][q] = Dn.s0[(int64_t)e * H + min(r0 + rb * 16 + ((lane >> 4) << 2) + q, H - 1)];
            v4i acc[2];
#pragma unroll
            for (int f = 0; f < NFD; ++f) {
                const int rb = f / KBD, kb = f % KBD;
                if (kb == 0) acc[0] = acc[1] = v4i{0, 0, 0, 0};
                const v4i b0 = *reinterpret_cast<const v4i*>(xl + kb * 1024 + lane * 16);
                const v4i b1 = *reinterpret_cast<const v4i*>(xl + (KBD + kb) * 1024 + lane * 16);
                acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(dring[f % DD], b0, acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(dring[f % DD], b1, acc[1], 0, 0, 0);
                if (f + DD < NFD) dring[f % DD] = dfrag(tn, f + DD);
                else if (tn + 1 < tiles_d) dring[f % DD] = dfrag(tn + 1, f + DD - NFD);
                __builtin_amdgcn_sched_barrier(0);
                if (kb == KBD - 1) {
                    const int nr = r0 + rb * 16 + ((lane >> 4) << 2);
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) {
                        const int j = tb * 16 + (lane & 15);
                        if (j >= gm) continue;
                        float* yrow = Dn.Y + (int64_t)(g0 + j) * Dn.ldy;
                        float4 v;
                        float* vp = &v.x;
#pragma unroll
                        for (int q = 0; q < 4; ++q) vp[q] = epilogue(acc[tb][q], ws[rb][q], xsd[tb]);
                        if (nr + 3 < H) {
                            *reinterpret_cast<float4*>(yrow + nr) = v;
                        } else {
#pragma unroll
                            for (int q = 0; q < 3; ++q)
                                if (nr + q < H) yrow[nr + q] = vp[q];
                        }
                    }
                }
            }
        }
    }
}

bool expert_fused_shape(int64_t H, int64_t I)
{
    auto ok = [](int64_t k) { return k == 512 || k == 1024 || k == 2048; };
    return ok(H) && ok(I);
}

template <int KBG, bool kSilu>
static void fused_for_kbd(int kbd, dim3 g, hipStream_t s, const ExpertArgs& G, const ExpertArgs& Dn)
{
    const dim3 b(256);
    if (kbd == 8) PF_LAUNCH((k_expert_fused<KBG, 8, kSilu>), g, b, 0, s, G, Dn);
    else if (kbd == 16) PF_LAUNCH((k_expert_fused<KBG, 16, kSilu>), g, b, 0, s, G, Dn);
    else PF_LAUNCH((k_expert_fused<KBG, 32, kSilu>), g, b, 0, s, G, Dn);
}

template <bool kSilu>
static void fused_for_kbg(int kbg, int kbd, dim3 g, hipStream_t s, const ExpertArgs& G, const ExpertArgs& Dn)
{
    if (kbg == 8) fused_for_kbd<8, kSilu>(kbd, g, s, G, Dn);
    else if (kbg == 16) fused_for_kbd<16, kSilu>(kbd, g, s, G, Dn);
    else fused_for_kbd<32, kSilu>(kbd, g, s, G, Dn);
}

hipError_t launch_expert_fused(const ExpertArgs& G, const ExpertArgs& Dn, hipStream_t s)
{
    if (!expert_fused_shape(G.K, G.N) || Dn.K != G.N || Dn.N != G.K || !G.W1 || !G.gather)
        return hipErrorInvalidValue;
    const dim3 g(G.E);
    if (G.act) fused_for_kbg<true>(G.K / 64, G.N / 64, g, s, G, Dn);
    else fused_for_kbg<false>(G.K / 64, G.N / 64, g, s, G, Dn);
    return hipGetLastError();
}

// The streaming form for K of 512, 1024 or 2048 and 16-byte aligned output
// rows; the piecewise form otherwise.
hipError_t launch_expert(const ExpertArgs& a, hipStream_t s)
{
    const dim3 b(256);
    const bool aligned = a.ldy % 4 == 0 && (reinterpret_cast<uintptr_t>(a.Y) & 15) == 0;
    if (aligned && (a.K == 512 || a.K == 1024 || a.K == 2048)) {
        // gate/up: 64 rows of each weight per workgroup; down: 64 RB rows, RB = 4
        // (2 at K = 2048), so that a wave streams 32 to 64 fragments
        ExpertArgs c = a;
        const int rb = a.W1 ? 1 : (a.K == 2048 ? 2 : 4);
        c.tiles_n = (a.N + 64 * rb - 1) / (64 * rb);
        const dim3 g(a.E * c.tiles_n);
        if (a.W1 && a.act) {
            if (a.K == 512) PF_LAUNCH((k_expert_stream<true, 1, 8, 8, true>), g, b, 0, s, c);
            else if (a.K == 1024) PF_LAUNCH((k_expert_stream<true, 1, 8, 16, true>), g, b, 0, s, c);
            else PF_LAUNCH((k_expert_stream<true, 1, 8, 32, true>), g, b, 0, s, c);
        } else if (a.W1) {
            if (a.K == 512) PF_LAUNCH((k_expert_stream<true, 1, 8, 8>), g, b, 0, s, c);
            else if (a.K == 1024) PF_LAUNCH((k_expert_stream<true, 1, 8, 16>), g, b, 0, s, c);
            else PF_LAUNCH((k_expert_stream<true, 1, 8, 32>), g, b, 0, s, c);
        } else {
            if (a.K == 512) PF_LAUNCH((k_expert_stream<false, 4, 16, 8>), g, b, 0, s, c);
            else if (a.K == 1024) PF_LAUNCH((k_expert_stream<false, 4, 16, 16>), g, b, 0, s, c);
            else PF_LAUNCH((k_expert_stream<false, 2, 16, 32>), g, b, 0, s, c);
        }
        return hipGetLastError();
    }
    const dim3 g(a.E * a.tiles_n);
    if (a.W1) PF_LAUNCH(k_expert<true>, g, b, 0, s, a);
    else PF_LAUNCH(k_expert<false>, g, b, 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weighted combine: out[t][j] = +0, then over the token's experts in ascending
// id out = fl(out + fl(w * y)).  The rows of eight experts at a time are loaded
// before any of them is added, so their loads are in flight together; the adds
// keep the ascending order.
constexpr int kCbBatch = 8;

__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ ypair,
                                                 const int* __restrict__ comb_row,
                                                 const float* __restrict__ comb_w, int k, int H,
                                                 float* __restrict__ out)
{
    const int t = blockIdx.x;
    float* o_row = out + (int64_t)t * H;
    const int* rows = comb_row + (int64_t)t * k;
    const float* wts = comb_w + (int64_t)t * k;
    if (((uintptr_t)o_row & 15) == 0 && (H & 3) == 0) {   // four outputs per lane, 16-byte accesses
        for (int j = threadIdx.x * 4; j < H; j += 1024) {
            float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            for (int r0 = 0; r0 < k; r0 += kCbBatch) {
                float4 y[kCbBatch];
                float wr[kCbBatch];
#pragma unroll
                for (int u = 0; u < kCbBatch; ++u) {
                    if (r0 + u < k) {
                        wr[u] = wts[r0 + u];
                        y[u] = *reinterpret_cast<const float4*>(ypair + (int64_t)rows[r0 + u] * H + j);
                    }
                }
#pragma unroll
                for (int u = 0; u < kCbBatch; ++u) {
                    if (r0 + u < k) {
                        o.x = o.x + wr[u] * y[u].x;
                        o.y = o.y + wr[u] * y[u].y;
                        o.z = o.z + wr[u] * y[u].z;
                        o.w = o.w + wr[u] * y[u].w;
                    }
                }
            }
            *reinterpret_cast<float4*>(o_row + j) = o;
        }
        return;
    }
    for (int j = threadIdx.x; j < H; j += 256) {
        float o = 0.0f;
        for (int r = 0; r < k; ++r) {
            const float c = wts[r] * ypair[(int64_t)rows[r] * H + j];
            o = o + c;
        }
        o_row[j] = o;
    }
}

hipError_t launch_combine(const float* ypair, const int* comb_row, const float* comb_w, int T,
                          int k, int H, float* out, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    PF_LAUNCH(k_combine, dim3(T), dim3(256), 0, s, ypair, comb_row, comb_w, k, H, out);
    return hipGetLastError();
}

}  // namespace pf
