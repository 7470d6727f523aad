// dense.hip — quantiser, per-token GEMV and the two MFMA products (gfx950).
//
// "Batched Prefill" (cellm), §The Solution: a weight row is loaded once and
// dotted against every token of the chunk; activations are quantised once per
// chunk; work is split over weight rows so that every weight byte is read once.
// Here a workgroup owns a band of weight rows, streams them from HBM with
// 128-bit loads straight into the MFMA operand registers, and takes the chunk's
// quantised tokens from LDS, where they are staged once per workgroup.
#include <cstring>

#include "device.hpp"
#include "expf_cr.hpp"
#include "kernels.hpp"
#include "problems.hpp"

namespace pf {

// ---------------------------------------------------------------------------
// Zero fill (workspace clearing without memset nodes).
__global__ __launch_bounds__(256) void k_fill_zero(v4i* p, size_t n16, int8_t* tail, int ntail)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = v4i{0, 0, 0, 0};
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s)
{
    if (bytes == 0) return hipSuccess;
    const size_t n16 = bytes / 16;
    const int ntail = (int)(bytes - n16 * 16);
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) blocks = 1;
    PF_LAUNCH(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<v4i*>(p), n16, reinterpret_cast<int8_t*>(p) + n16 * 16,
                       ntail);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-token quantisation: one workgroup per token row.  amax is an exact
// maximum (order-free); the scale and every code follow the per-token
// definition bit for bit.
// r = fl(silu(g) * u) elementwise (the gated SiLU's row).
__device__ __forceinline__ float4 gated(float4 g, float4 u)
{
    return float4{silu_cr(g.x) * u.x, silu_cr(g.y) * u.y, silu_cr(g.z) * u.z, silu_cr(g.w) * u.w};
}

// With gate != null the row quantised is gated(gate, x), evaluated again in the
// second pass (the same bits).
__device__ __forceinline__ void quantize_row(const float* __restrict__ x, int K,
                                             int8_t* __restrict__ q, float* __restrict__ scale,
                                             const float* __restrict__ gate = nullptr)
{
    const float4* row = reinterpret_cast<const float4*>(x);
    const float4* grow = reinterpret_cast<const float4*>(gate);
    int* qrow = reinterpret_cast<int*>(q);
    const int n4 = K >> 2;
    float amax = 0.0f;
    for (int i = threadIdx.x; i < n4; i += 256) {
        const float4 v = gate ? gated(grow[i], row[i]) : row[i];
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    amax = wave_max(amax);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) *scale = s;
    for (int i = threadIdx.x; i < n4; i += 256) {
        int packed = 0;
        if (s != 0.0f) {
            const float4 v = gate ? gated(grow[i], row[i]) : row[i];
            packed = (quant_code(v.x, s) & 0xff) | ((quant_code(v.y, s) & 0xff) << 8) |
                     ((quant_code(v.z, s) & 0xff) << 16) | ((quant_code(v.w, s) & 0xff) << 24);
        }
        qrow[i] = packed;
    }
}

// Rows of at most 1024 values, one wave per row and four rows per workgroup:
// lane l holds the row's float4 pieces l + 64 u in registers, the maximum is a
// wave reduction (no workgroup barrier), and the codes come from the registers.
// Same arithmetic as quant_row_regs.
template <int U>
__global__ __launch_bounds__(256) void k_quantize_rows(const float* __restrict__ x, int64_t ldx, int M,
                                                       int K, int8_t* __restrict__ q,
                                                       float* __restrict__ scale)
{
    const int lane = threadIdx.x & 63;
    const int t = (int)blockIdx.x * 4 + ((int)threadIdx.x >> 6);
    if (t >= M) return;                                  // the whole wave
    const int n4 = K >> 2;
    const float4* row = reinterpret_cast<const float4*>(x + (int64_t)t * ldx);
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = row[min(lane + 64 * u, n4 - 1)];
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (lane + 64 * u < n4)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    amax = wave_max(amax);
    const float s = amax / 127.0f;
    if (lane == 0) scale[t] = s;
    int* qrow = reinterpret_cast<int*>(q + (int64_t)t * K);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = lane + 64 * u;
        if (i >= n4) continue;
        int packed = 0;
        if (s != 0.0f)
            packed = (quant_code(v[u].x, s) & 0xff) | ((quant_code(v[u].y, s) & 0xff) << 8) |
                     ((quant_code(v[u].z, s) & 0xff) << 16) | ((quant_code(v[u].w, s) & 0xff) << 24);
        qrow[i] = packed;
    }
}

// M rows of x [M][ldx]: rows of at most 1024 values one wave each (the MoE's
// 5120 rows of 512: 11 -> 5.7 us; rows of 2048 took 4.8 -> 5.9 us, so longer
// rows stay with a workgroup each); longer rows through the quantisation-step
// kernel with one pair (rows held in registers up to 16384 values, two passes
// over the row beyond).
hipError_t launch_quantize(const float* x, int64_t ldx, int M, int K, int8_t* q, float* scale,
                           hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    const int n4 = K >> 2;
    if (n4 <= 256) {
        const dim3 g((M + 3) / 4), b(256);
        if (n4 <= 64) PF_LAUNCH(k_quantize_rows<1>, g, b, 0, s, x, ldx, M, K, q, scale);
        else if (n4 <= 128) PF_LAUNCH(k_quantize_rows<2>, g, b, 0, s, x, ldx, M, K, q, scale);
        else PF_LAUNCH(k_quantize_rows<4>, g, b, 0, s, x, ldx, M, K, q, scale);
        return hipGetLastError();
    }
    QuantStep S;
    std::memset(&S, 0, sizeof(S));
    S.npairs = 1;
    S.K = K;
    S.total_rows = M;
    S.pair[0].src = x;
    S.pair[0].ld = ldx;
    S.pair[0].q = q;
    S.pair[0].s = scale;
    return launch_quantize_step(S, s);
}

// The token rows of several chunks in one launch (one workgroup per row).
__device__ __forceinline__ void rebuild_row(const QuantPair& P, int t, int K)
{
    // h[n] = epilogue(sum over splits of part[s][t][n], ws[n], as[t]); integer
    // sums, so the split order does not matter.
    const float as = P.as[t];
    const int4* prow = reinterpret_cast<const int4*>(P.part + (int64_t)t * K);
    float4* hrow = reinterpret_cast<float4*>(P.h + (int64_t)t * P.ldh);
    float* yrow = P.y ? P.y + (int64_t)t * K : nullptr;    // 4-byte aligned only
    const int64_t sstride = P.part_stride / 4;
    for (int i = threadIdx.x; i < (K >> 2); i += 256) {
        int4 v = prow[i];
        for (int sp = 1; sp < P.splits; ++sp) {
            const int4 w = prow[i + sp * sstride];
            v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
        }
        const float* ws = P.ws + 4 * i;      // scales need only 4-byte alignment
        float4 h;
        h.x = epilogue(v.x, ws[0], as);
        h.y = epilogue(v.y, ws[1], as);
        h.z = epilogue(v.z, ws[2], as);
        h.w = epilogue(v.w, ws[3], as);
        hrow[i] = h;
        if (yrow) {
            yrow[4 * i] = h.x;
            yrow[4 * i + 1] = h.y;
            yrow[4 * i + 2] = h.z;
            yrow[4 * i + 3] = h.w;
        }
    }
}

// A row of at most 1024 U values with the values held in registers (U
// float4 pieces per thread, pieces i = threadIdx.x + 256 u): every load of the
// row is issued before any is used (the split partials four splits at a time
// up to U = 4), and the codes come from the registers, so the row is read once.
// Same arithmetic as rebuild_row followed by quantize_row.
template <int U, bool kGated>
__device__ __forceinline__ void quant_row_regs(const QuantPair& P, int t, int K)
{
    const int n4 = K >> 2;
    int idx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) idx[u] = min((int)threadIdx.x + 256 * u, n4 - 1);
    float4 v[U];
    if (P.part) {
        const int4* prow = reinterpret_cast<const int4*>(P.part + (int64_t)t * K);
        const int64_t sstride = P.part_stride / 4;
        int4 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = prow[idx[u]];
        constexpr int SB = U <= 4 ? 4 : 1;          // splits loaded together
        for (int sp0 = 1; sp0 < P.splits; sp0 += SB) {
            int4 w[U][SB];
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int64_t off = (int64_t)min(sp0 + j, P.splits - 1) * sstride;
#pragma unroll
                for (int u = 0; u < U; ++u) w[u][j] = prow[idx[u] + off];
            }
#pragma unroll
            for (int j = 0; j < SB; ++j)
                if (sp0 + j < P.splits)
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        a[u].x += w[u][j].x; a[u].y += w[u][j].y; a[u].z += w[u][j].z; a[u].w += w[u][j].w;
                    }
        }
        const float as = P.as[t];
        float4* hrow = P.h ? reinterpret_cast<float4*>(P.h + (int64_t)t * P.ldh) : nullptr;
        float* yrow = P.y ? P.y + (int64_t)t * K : nullptr;    // 4-byte aligned only
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = (int)threadIdx.x + 256 * u;
            const float* ws = P.ws + 4 * idx[u];
            v[u].x = epilogue(a[u].x, ws[0], as);
            v[u].y = epilogue(a[u].y, ws[1], as);
            v[u].z = epilogue(a[u].z, ws[2], as);
            v[u].w = epilogue(a[u].w, ws[3], as);
            if (i < n4) {
                if (hrow) hrow[i] = v[u];
                if (yrow) {
                    yrow[4 * i] = v[u].x;
                    yrow[4 * i + 1] = v[u].y;
                    yrow[4 * i + 2] = v[u].z;
                    yrow[4 * i + 3] = v[u].w;
                }
            }
        }
        if (!P.q) return;
    } else {
        const float4* row = reinterpret_cast<const float4*>(P.src + (int64_t)t * P.ld);
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = row[idx[u]];
        if (kGated) {
            const float4* grow = reinterpret_cast<const float4*>(P.gate + (int64_t)t * P.ld);
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = gated(grow[idx[u]], v[u]);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
        if ((int)threadIdx.x + 256 * u < n4)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    amax = wave_max(amax);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) P.s[t] = s;
    int* qrow = reinterpret_cast<int*>(P.q + (int64_t)t * K);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = (int)threadIdx.x + 256 * u;
        if (i >= n4) continue;
        int packed = 0;
        if (s != 0.0f)
            packed = (quant_code(v[u].x, s) & 0xff) | ((quant_code(v[u].y, s) & 0xff) << 8) |
                     ((quant_code(v[u].z, s) & 0xff) << 16) | ((quant_code(v[u].w, s) & 0xff) << 24);
        qrow[i] = packed;
    }
}

// Rows of up to 4096 values (kLong = false) or longer (kLong, with more
// registers per thread; a separate kernel so the short rows keep their
// occupancy).
template <bool kLong, bool kGated>
__global__ __launch_bounds__(256) void k_quantize_step(QuantStep S)
{
    const int bid = blockIdx.x;
    int pi = 0;
#pragma unroll
    for (int q = 1; q < kMaxQuant; ++q)
        if (q < S.npairs && bid >= S.pair[q].row0) pi = q;
    const QuantPair& P = S.pair[pi];
    const int t = bid - P.row0;
    const int n4 = S.K >> 2;
    if (kLong) {
        if (n4 <= 2048) return quant_row_regs<8, kGated>(P, t, S.K);
        if (n4 <= 3072) return quant_row_regs<12, kGated>(P, t, S.K);
        if (n4 <= 4096) return quant_row_regs<16, kGated>(P, t, S.K);
    } else {
        if (n4 <= 256) return quant_row_regs<1, kGated>(P, t, S.K);
        if (n4 <= 512) return quant_row_regs<2, kGated>(P, t, S.K);
        if (n4 <= 1024) return quant_row_regs<4, kGated>(P, t, S.K);
    }
    if (P.part) {
        rebuild_row(P, t, S.K);
        if (!P.q) return;
        // each thread re-reads only the elements it wrote itself
        quantize_row(P.h + (int64_t)t * P.ldh, S.K, P.q + (int64_t)t * S.K, P.s + t);
        return;
    }
    quantize_row(P.src + (int64_t)t * P.ld, S.K, P.q + (int64_t)t * S.K, P.s + t,
                 kGated ? P.gate + (int64_t)t * P.ld : nullptr);
}

hipError_t launch_quantize_gated(const float* up, const float* gate, int64_t ld, int M, int K,
                                 int8_t* q, float* scale, hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    QuantStep S;
    std::memset(&S, 0, sizeof(S));
    S.npairs = 1;
    S.K = K;
    S.total_rows = M;
    S.pair[0].src = up;
    S.pair[0].gate = gate;
    S.pair[0].ld = ld;
    S.pair[0].q = q;
    S.pair[0].s = scale;
    return launch_quantize_step(S, s);
}

hipError_t launch_quantize_step(const QuantStep& S, hipStream_t s)
{
    if (S.total_rows <= 0) return hipSuccess;
    // gated rows (every pair of a launch alike) in their own instantiations, so
    // that the plain ones carry no call
    const bool gated = S.pair[0].gate != nullptr;
    for (int i = 1; i < S.npairs; ++i)
        if ((S.pair[i].gate != nullptr) != gated) return hipErrorInvalidValue;
    const dim3 g(S.total_rows), b(256);
    if (gated) {
        if (S.K > 4096) PF_LAUNCH((k_quantize_step<true, true>), g, b, 0, s, S);
        else PF_LAUNCH((k_quantize_step<false, true>), g, b, 0, s, S);
    } else {
        if (S.K > 4096) PF_LAUNCH((k_quantize_step<true, false>), g, b, 0, s, S);
        else PF_LAUNCH((k_quantize_step<false, false>), g, b, 0, s, S);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-token GEMV (M = 1): a workgroup owns 16 weight rows, NW waves of 16 / NW
// rows each; each lane streams 16-byte pieces of its wave's rows, multiplies
// with v_dot4_i32_i8 and the wave reduces the int32 sums.  The token's 16-byte
// pieces are re-read from L1/L2 per row group.  The weights are loaded as
// non-temporal (each byte is used once per token): 4096 x 4096 kernel 6.2 ->
// 5.3 us, the 350M stack's per-token mode 219.7 -> 215.7 ms; a copy of the
// token per workgroup in LDS was slower.
constexpr int kGemvTile = 16;

template <int NW>
__global__ __launch_bounds__(64 * NW) void k_gemv(GemmSet set)
{
    constexpr int R = kGemvTile / NW;                    // rows per wave
    const GemmProb P = find_prob(set, blockIdx.x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nbase = (blockIdx.x - P.tile_begin) * kGemvTile + wave * R;
    const int nchunks = P.K >> 4;
    const int8_t* wrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int n = min(nbase + r, P.N - 1);
        wrow[r] = P.W + (int64_t)n * P.K;
    }
    int acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0;
#pragma unroll 4
    for (int c = lane; c < nchunks; c += 64) {
        const v4i qv = ld16(P.X + c * 16);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const v4i wv = ld16_nt(wrow[r] + c * 16);
            acc[r] = __builtin_amdgcn_sdot4(wv.x, qv.x, acc[r], false);
            acc[r] = __builtin_amdgcn_sdot4(wv.y, qv.y, acc[r], false);
            acc[r] = __builtin_amdgcn_sdot4(wv.z, qv.z, acc[r], false);
            acc[r] = __builtin_amdgcn_sdot4(wv.w, qv.w, acc[r], false);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
    if (lane == 0) {
        const float xs = P.xs[0];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = nbase + r;
            if (n < P.N) store_out(P, 0, n, epilogue(acc[r], P.ws[n], xs));
        }
    }
}

// One row per wave: sixteen waves per workgroup keep four times the loads in
// flight per compute unit of four waves of four rows (4096 x 4096: 11.2 ->
// 8.7 us per call back to back, eight waves of two rows 8.9 us).
constexpr int kGemvWaves = 16;

hipError_t launch_gemv(const GemmSet& set, hipStream_t s)
{
    if (set.total_tiles <= 0) return hipSuccess;
    PF_LAUNCH(k_gemv<kGemvWaves>, dim3(set.total_tiles), dim3(64 * kGemvWaves), 0, s, set);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Skinny product (M <= 64): v_mfma_i32_16x16x64_i8 with the weights as the A
// operand (lane l holds 16 bytes of weight row l%16) and the tokens as B (lane l
// holds the same 16 k positions of token l%16).  A workgroup owns 64 weight rows
// (16 per wave) and all M tokens over its K range.  The tokens are staged in LDS
// one piece of KP k-blocks (of 64 bytes) at a time and shared by the four waves;
// each lane loads its weight fragments straight from HBM into registers, one
// piece ahead of the MFMAs (the four lanes l, l+16, l+32, l+48 read 64
// contiguous bytes of a row).  LDS holds two token pieces: while the waves
// multiply piece p, piece p+1 travels from L2 into registers and is written to
// the other buffer.  When a launch has too few 64-row tiles to fill the chip,
// the K range is also split across workgroups: each writes its int32 partial
// tile to the workspace and k_split_reduce sums the partials (integer sums,
// so the bits do not depend on the split) and applies the epilogue.
constexpr int kSkRows = 64;

template <int TB, int KP>
__device__ __forceinline__ void skinny_tile(const GemmProb& P, int local)
{
    constexpr int kStride = KP * 64 + 16;               // LDS bytes per token row
    constexpr int kChunks = 16 * TB * KP * 4;            // 16-byte chunks per token piece
    constexpr int kPerThread = (kChunks + 255) / 256;
    __shared__ __attribute__((aligned(16))) int8_t xl[2][16 * TB * kStride];
    const int split = local % P.splits;
    const int tn = local / P.splits;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw0 = tn * kSkRows + wave * 16;
    const int nkb = P.K >> 6;
    const int kb0 = split * P.kb_per_split;
    const int kb1 = min(kb0 + P.kb_per_split, nkb);
    const int npieces = (kb1 - kb0 + KP - 1) / KP;
    const int koff = (lane >> 4) << 4;
    const int8_t* wp = P.W + (int64_t)min(nw0 + (lane & 15), P.N - 1) * P.K + koff;
    const int boff = (lane & 15) * kStride + koff;

    // token piece staging: thread chunk c -> token c / (4 KP), 16-byte column c % (4 KP)
    auto xload = [&](int kp, int npc, v4i (&r)[kPerThread]) {
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const int c = tid + 256 * u;
            const int t = c / (4 * KP), col = c % (4 * KP);
            r[u] = v4i{0, 0, 0, 0};
            if (c < kChunks && t < P.M && col < 4 * npc)
                r[u] = ld16(P.X + (int64_t)t * P.ldx + (int64_t)kp * 64 + col * 16);
        }
    };
    auto xstore = [&](int buf, const v4i (&r)[kPerThread]) {
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const int c = tid + 256 * u;
            if (c < kChunks) st16(&xl[buf][(c / (4 * KP)) * kStride + (c % (4 * KP)) * 16], r[u]);
        }
    };
    auto wload = [&](int kp, int npc, v4i (&a)[KP]) {
#pragma unroll
        for (int i = 0; i < KP; ++i)
            if (i < npc) a[i] = ld16(wp + (int64_t)(kp + i) * 64);
    };

    v4i acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = v4i{0, 0, 0, 0};
    v4i a0[KP], a1[KP], xr[kPerThread];

    int npc = min(KP, kb1 - kb0);
    wload(kb0, npc, a0);
    xload(kb0, npc, xr);
    xstore(0, xr);
    for (int p = 0; p < npieces; ++p) {
        const int kp = kb0 + p * KP;
        const int npc_next = p + 1 < npieces ? min(KP, kb1 - kp - KP) : 0;
        if (npc_next > 0) {
            wload(kp + KP, npc_next, a1);
            xload(kp + KP, npc_next, xr);
        }
        __syncthreads();
        const int8_t* xb = xl[p & 1] + boff;
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            if (i < npc) {
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const v4i b = *reinterpret_cast<const v4i*>(xb + tb * 16 * kStride + i * 64);
                    acc[tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[i], b, acc[tb], 0, 0, 0);
                }
            }
        }
        if (npc_next > 0) {
            xstore((p + 1) & 1, xr);
#pragma unroll
            for (int i = 0; i < KP; ++i) a0[i] = a1[i];
        }
        npc = npc_next;
    }

    // Lane l holds rows nr .. nr+3 of token column l%16 in each token block.
    const int nr = nw0 + ((lane >> 4) << 2);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int t = tb * 16 + (lane & 15);
        if (t >= P.M) continue;
        if (P.splits == 1) {
            const float xs = P.xs[t];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (nr + r < P.N) store_out(P, t, nr + r, epilogue(acc[tb][r], P.ws[nr + r], xs));
        } else {
            int* part = P.acc + (int64_t)split * P.acc_split + (int64_t)t * P.acc_ld;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (nr + r < P.N) part[nr + r] = acc[tb][r];
        }
    }
}

template <int TB, int KP>
__global__ __launch_bounds__(256) void k_gemm_skinny(GemmSet set)
{
    const GemmProb P = find_prob(set, blockIdx.x);
    skinny_tile<TB, KP>(P, blockIdx.x - P.tile_begin);
}


// Sum of the split partials and the epilogue.  A workgroup takes 1024 outputs
// of the flattened M x N result (tile_begin counts such blocks), a thread four
// consecutive ones.  When N, the row strides and the bases are multiples of
// four elements (16 bytes), a thread's four outputs lie in one row and move as
// 16-byte loads and stores, four splits' loads in flight at once; otherwise it
// takes them one at a time.  The sums are integer sums, so the bits do not
// depend on their order.
constexpr int kReduceBlock = 1024;

__global__ __launch_bounds__(256) void k_split_reduce(GemmSet set)
{
    const GemmProb P = find_prob(set, blockIdx.x);
    const int64_t total = (int64_t)P.M * P.N;
    const int64_t i0 = ((int64_t)(blockIdx.x - P.tile_begin) * 256 + threadIdx.x) * 4;
    if (i0 >= total) return;
    const bool vec = (P.N & 3) == 0 && (P.acc_ld & 3) == 0 && (P.acc_split & 3) == 0 &&
                     ((uintptr_t)P.acc & 15) == 0 && ((uintptr_t)P.Y & 15) == 0 && (P.ldy & 3) == 0 &&
                     (!P.Y2 || (((uintptr_t)P.Y2 & 15) == 0 && (P.ldy2 & 3) == 0));
    if (vec) {
        const int t = (int)(i0 / P.N), n = (int)(i0 - (int64_t)t * P.N);
        const int* a = P.acc + (int64_t)t * P.acc_ld + n;
        v4i v = v4i{0, 0, 0, 0};
        int sp = 0;
        for (; sp + 4 <= P.splits; sp += 4) {
            v4i q[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) q[u] = *reinterpret_cast<const v4i*>(a + (int64_t)(sp + u) * P.acc_split);
#pragma unroll
            for (int u = 0; u < 4; ++u) v += q[u];
        }
        for (; sp < P.splits; ++sp) v += *reinterpret_cast<const v4i*>(a + (int64_t)sp * P.acc_split);
        const float xs = P.xs[t];
        float4 o;
        o.x = epilogue(v[0], P.ws[n], xs);
        o.y = epilogue(v[1], P.ws[n + 1], xs);
        o.z = epilogue(v[2], P.ws[n + 2], xs);
        o.w = epilogue(v[3], P.ws[n + 3], xs);
        *reinterpret_cast<float4*>(P.Y + (int64_t)t * P.ldy + n) = o;
        if (P.Y2) *reinterpret_cast<float4*>(P.Y2 + (int64_t)t * P.ldy2 + n) = o;
        return;
    }
    for (int r = 0; r < 4; ++r) {
        const int64_t idx = i0 + r;
        if (idx >= total) break;
        const int t = (int)(idx / P.N), n = (int)(idx - (int64_t)t * P.N);
        const int* a = P.acc + (int64_t)t * P.acc_ld + n;
        int v = 0;
        for (int sp = 0; sp < P.splits; ++sp) v += a[(int64_t)sp * P.acc_split];
        store_out(P, t, n, epilogue(v, P.ws[n], P.xs[t]));
    }
}

hipError_t launch_split_reduce(const GemmSet& set, hipStream_t s)
{
    // reduce launch over the split problems only; problems without splits get
    // no blocks (find_prob never selects them: their tile_begin equals the
    // next problem's)
    GemmSet r = set;
    int begin = 0;
    for (int i = 0; i < r.nprob; ++i) {
        r.p[i].tile_begin = begin;
        if (r.p[i].splits > 1) begin += (int)(((int64_t)r.p[i].M * r.p[i].N + kReduceBlock - 1) / kReduceBlock);
    }
    if (begin == 0) return hipSuccess;
    r.total_tiles = begin;
    PF_LAUNCH(k_split_reduce, dim3(begin), dim3(256), 0, s, r);
    return hipGetLastError();
}

// Token pieces of 8 k-blocks (512 bytes): with the weight double buffer that is
// 32 KB of weights in flight per workgroup at four workgroups per compute unit.
constexpr int kSkPiece = 8;

#define PF_SKINNY_CASES(KERNEL, ARG)                                                   \
    switch (token_blocks) {                                                            \
        case 1: PF_LAUNCH((KERNEL<1, kSkPiece>), g, b, 0, s, ARG); break;      \
        case 2: PF_LAUNCH((KERNEL<2, kSkPiece>), g, b, 0, s, ARG); break;      \
        case 3: PF_LAUNCH((KERNEL<3, kSkPiece>), g, b, 0, s, ARG); break;      \
        case 4: PF_LAUNCH((KERNEL<4, kSkPiece>), g, b, 0, s, ARG); break;      \
        default: return hipErrorInvalidValue;                                          \
    }

hipError_t launch_gemm_skinny(const GemmSet& set, int token_blocks, hipStream_t s)
{
    if (set.total_tiles <= 0) return hipSuccess;
    if (token_blocks < 1 || token_blocks > 4) return hipErrorInvalidValue;
    const dim3 g(set.total_tiles), b(256);
    PF_SKINNY_CASES(k_gemm_skinny, set)
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_reduce(set, s);
}

}  // namespace pf
