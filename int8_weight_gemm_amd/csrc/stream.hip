// stream.hip — the weight-streaming int8 product for chunks of up to 64 tokens.
//
// "Batched Prefill" (cellm), §The arithmetic and §The Solution: at chunk sizes
// of tens of tokens the product is bound by the weight stream, so the kernel's
// job is to keep HBM busy.  Each workgroup walks its share of 64-row tiles as one
// continuous pipeline of stages; a stage is KP k-blocks (of 64 bytes) of the
// tile's 64 weight rows plus the same k-blocks of the chunk's tokens.  Both are
// copied from global memory straight into LDS with global_load_lds_dwordx4
// (gfx950): no registers are tied up in flight, so NS - 1 stages are in flight
// while the waves multiply the oldest one.  Lane l of a DMA instruction lands
// at LDS base + 16 l; the addresses are chosen so that those 16 bytes are lane
// l's operand of v_mfma_i32_16x16x64_i8 (weight row l%16 as A, token l%16 as
// B, k positions 16*(l/16) .. +16 of the k-block), read back with one
// conflict-free ds_read_b128 per operand.  The pipeline runs across tile
// boundaries, so it drains only once per workgroup.
#include "device.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"
#include "problems.hpp"

namespace pf {

__device__ __forceinline__ GemmProb stream_prob(const StackStep& S, int tile, int& local)
{
    return step_prob(S, tile, local);
}

template <int TB, int KP, int NS>
__global__ __launch_bounds__(256) void k_gemm_stream(StackStep S, int ntiles)
{
    constexpr int kWBytes = 4 * KP * 1024;       // weights of one stage (4 waves x KP k-blocks)
    constexpr int kXBytes = TB * KP * 1024;      // tokens of one stage
    constexpr int kScales = kWBytes + kXBytes;   // 64 weight-row scales, then 64 token scales
    constexpr int kStage = kScales + 512;
    constexpr int kXPerWave = TB * KP / 4;       // token DMA instructions per wave and stage
    // DMA instructions per wave and stage; waves 0 and 1 also copy the scales
    constexpr int kLw = KP + kXPerWave;
    constexpr int kLs = kLw + 1;
    static_assert((TB * KP) % 4 == 0, "token DMAs must split evenly over the waves");
    static_assert(kLs * (NS - 2) <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(16))) int8_t lds[NS * kStage];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int G = gridDim.x;
    const int my_tiles = (ntiles - (int)blockIdx.x + G - 1) / G;
    if (my_tiles <= 0) return;
    const int nkb = S.K >> 6;
    const int spt = (nkb + KP - 1) / KP;         // stages per tile
    const int total = my_tiles * spt;
    // copies: four consecutive lanes per row (lane l: row l / 4, piece
    // (l % 4) ^ ((l / 8) % 4)); the operand of lane l (row l % 16, piece l / 16)
    // is then at `lofs` in its fragment (conflict-free)
    const int crow = lane >> 2;
    const int koff = ((lane & 3) ^ ((lane >> 3) & 3)) << 4;
    const int lofs = (lane & 15) * 64 + (((lane >> 4) ^ ((lane >> 1) & 3)) << 4);

    // ---- issue side: the tile whose stages are being loaded
    int itile = -1;
    const int8_t* iw = nullptr;                  // this lane's weight row (+koff)
    const int8_t* ix[kXPerWave];                 // token row of each token DMA (+koff)
    const float* isc = nullptr;                  // wave 0: weight-row scale, wave 1: token scale
    auto issue = [&](int g) {
        if (g >= total) return;
        const int t = g / spt, piece = g - t * spt;
        if (t != itile) {
            itile = t;
            int local;
            const GemmProb P = stream_prob(S, (int)blockIdx.x + t * G, local);
            const int n = min(local * 64 + wave * 16 + crow, P.N - 1);
            iw = P.W + (int64_t)n * P.K + koff;
#pragma unroll
            for (int u = 0; u < kXPerWave; ++u) {
                const int q = wave + 4 * u, tb = q / KP;
                const int tok = tb * 16 + crow;
                ix[u] = P.X + (int64_t)(tok < P.M ? tok : 0) * P.ldx + koff;
            }
            if (wave == 0) isc = P.ws + min(local * 64 + lane, P.N - 1);
            if (wave == 1) isc = P.xs + min(lane, P.M - 1);
        }
        int8_t* base = lds + (g % NS) * kStage;
        const int kb0 = piece * KP;
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int kb = min(kb0 + i, nkb - 1);    // a ragged last piece repeats a valid block
            dma16(iw + (int64_t)kb * 64, base + (wave * KP + i) * 1024);
        }
#pragma unroll
        for (int u = 0; u < kXPerWave; ++u) {
            const int q = wave + 4 * u, i = q % KP;
            const int kb = min(kb0 + i, nkb - 1);
            dma16(ix[u] + (int64_t)kb * 64, base + kWBytes + q * 1024);
        }
        if (wave < 2) dma4(isc, base + kScales + wave * 256);
    };

    // ---- compute side
    v4i acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = v4i{0, 0, 0, 0};

#pragma unroll
    for (int g = 0; g < NS - 1; ++g) issue(g);

    for (int g = 0; g < total; ++g) {
        const int ahead = min(NS - 2, total - 1 - g);   // stages issued after stage g
        if (ahead <= 0) wait_vmcnt<0>();
        else if (wave < 2) {
            if (ahead == 1) wait_vmcnt<kLs>();
            else if (ahead == 2) wait_vmcnt<2 * kLs>();
            else wait_vmcnt<3 * kLs>();
        } else {
            if (ahead == 1) wait_vmcnt<kLw>();
            else if (ahead == 2) wait_vmcnt<2 * kLw>();
            else wait_vmcnt<3 * kLw>();
        }
        stage_barrier();                              // stage g complete; stage g-1 consumed
        const int t = g / spt, piece = g - t * spt;
        int local;
        const GemmProb P = stream_prob(S, (int)blockIdx.x + t * G, local);
        const int nr = local * 64 + wave * 16 + ((lane >> 4) << 2);
        issue(g + NS - 1);
        const int npc = min(KP, nkb - piece * KP);
        const int8_t* base = lds + (g % NS) * kStage;
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            if (i < npc) {
                const v4i a = *reinterpret_cast<const v4i*>(base + (wave * KP + i) * 1024 + lofs);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const v4i b = *reinterpret_cast<const v4i*>(base + kWBytes + (tb * KP + i) * 1024 + lofs);
                    acc[tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[tb], 0, 0, 0);
                }
            }
        }
        if (piece == spt - 1) {
            // the scales came with every stage of this tile; use the current one
            const float* wsl = reinterpret_cast<const float*>(base + kScales) + wave * 16 + ((lane >> 4) << 2);
            const float* xsl = reinterpret_cast<const float*>(base + kScales + 256);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int tok = tb * 16 + (lane & 15);
                if (tok < P.M) {
                    const float xs = xsl[tok];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (nr + r < P.N) store_out(P, tok, nr + r, epilogue(acc[tb][r], wsl[r], xs));
                }
                acc[tb] = v4i{0, 0, 0, 0};
            }
        }
    }
}

// Workgroups: one per 64-row tile, at most two per compute unit (the LDS of a
// workgroup holds NS stages).
hipError_t launch_gemm_stream(const StackStep& S, int token_blocks, hipStream_t s)
{
    const int ntiles = S.npairs * S.tile_off[S.nproj];
    if (ntiles <= 0) return hipSuccess;
    const int grid = ntiles < 512 ? ntiles : 512;
    const dim3 g(grid), b(256);
    switch (token_blocks) {
        case 1: PF_LAUNCH((k_gemm_stream<1, 4, 4>), g, b, 0, s, S, ntiles); break;
        case 2: PF_LAUNCH((k_gemm_stream<2, 4, 3>), g, b, 0, s, S, ntiles); break;
        case 3: PF_LAUNCH((k_gemm_stream<3, 4, 3>), g, b, 0, s, S, ntiles); break;
        case 4: PF_LAUNCH((k_gemm_stream<4, 4, 3>), g, b, 0, s, S, ntiles); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// One stage's MFMA operands (KP k-blocks): the weight fragment of each k-block
// (at wa + 1 KB i) and the token fragments of TB token blocks (at
// xa + (16 tb + i) KB), in one assembly block.
template <int TB, int KP>
struct StageFrags {
    v4i a[KP];
    v4i b[TB][KP];
};

template <int TB, int KP>
__device__ __forceinline__ void lds_stage(StageFrags<TB, KP>& f, uint32_t wa, uint32_t xa);

template <>
__device__ __forceinline__ void lds_stage<1, 2>(StageFrags<1, 2>& f, uint32_t wa, uint32_t xa)
{
    asm volatile(
        "ds_read_b128 %0, %4 offset:0\n"
        "ds_read_b128 %1, %5 offset:0\n"
        "ds_read_b128 %2, %4 offset:1024\n"
        "ds_read_b128 %3, %5 offset:1024\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f.a[0]), "=&v"(f.b[0][0]), "=&v"(f.a[1]), "=&v"(f.b[0][1])
        : "v"(wa), "v"(xa));
}

template <>
__device__ __forceinline__ void lds_stage<2, 2>(StageFrags<2, 2>& f, uint32_t wa, uint32_t xa)
{
    asm volatile(
        "ds_read_b128 %0, %6 offset:0\n"
        "ds_read_b128 %1, %7 offset:0\n"
        "ds_read_b128 %2, %7 offset:16384\n"
        "ds_read_b128 %3, %6 offset:1024\n"
        "ds_read_b128 %4, %7 offset:1024\n"
        "ds_read_b128 %5, %7 offset:17408\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f.a[0]), "=&v"(f.b[0][0]), "=&v"(f.b[1][0]), "=&v"(f.a[1]),
          "=&v"(f.b[0][1]), "=&v"(f.b[1][1])
        : "v"(wa), "v"(xa));
}

template <>
__device__ __forceinline__ void lds_stage<3, 2>(StageFrags<3, 2>& f, uint32_t wa, uint32_t xa)
{
    asm volatile(
        "ds_read_b128 %0, %8 offset:0\n"
        "ds_read_b128 %1, %9 offset:0\n"
        "ds_read_b128 %2, %9 offset:16384\n"
        "ds_read_b128 %3, %9 offset:32768\n"
        "ds_read_b128 %4, %8 offset:1024\n"
        "ds_read_b128 %5, %9 offset:1024\n"
        "ds_read_b128 %6, %9 offset:17408\n"
        "ds_read_b128 %7, %9 offset:33792\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f.a[0]), "=&v"(f.b[0][0]), "=&v"(f.b[1][0]), "=&v"(f.b[2][0]),
          "=&v"(f.a[1]), "=&v"(f.b[0][1]), "=&v"(f.b[1][1]), "=&v"(f.b[2][1])
        : "v"(wa), "v"(xa));
}

template <>
__device__ __forceinline__ void lds_stage<4, 2>(StageFrags<4, 2>& f, uint32_t wa, uint32_t xa)
{
    asm volatile(
        "ds_read_b128 %0, %10 offset:0\n"
        "ds_read_b128 %1, %11 offset:0\n"
        "ds_read_b128 %2, %11 offset:16384\n"
        "ds_read_b128 %3, %11 offset:32768\n"
        "ds_read_b128 %4, %11 offset:49152\n"
        "ds_read_b128 %5, %10 offset:1024\n"
        "ds_read_b128 %6, %11 offset:1024\n"
        "ds_read_b128 %7, %11 offset:17408\n"
        "ds_read_b128 %8, %11 offset:33792\n"
        "ds_read_b128 %9, %11 offset:50176\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f.a[0]), "=&v"(f.b[0][0]), "=&v"(f.b[1][0]), "=&v"(f.b[2][0]),
          "=&v"(f.b[3][0]), "=&v"(f.a[1]), "=&v"(f.b[0][1]), "=&v"(f.b[1][1]),
          "=&v"(f.b[2][1]), "=&v"(f.b[3][1])
        : "v"(wa), "v"(xa));
}

template <>
__device__ __forceinline__ void lds_stage<1, 4>(StageFrags<1, 4>& f, uint32_t wa, uint32_t xa)
{
    asm volatile(
        "ds_read_b128 %0, %8 offset:0\n"
        "ds_read_b128 %1, %9 offset:0\n"
        "ds_read_b128 %2, %8 offset:1024\n"
        "ds_read_b128 %3, %9 offset:1024\n"
        "ds_read_b128 %4, %8 offset:2048\n"
        "ds_read_b128 %5, %9 offset:2048\n"
        "ds_read_b128 %6, %8 offset:3072\n"
        "ds_read_b128 %7, %9 offset:3072\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f.a[0]), "=&v"(f.b[0][0]), "=&v"(f.a[1]), "=&v"(f.b[0][1]),
          "=&v"(f.a[2]), "=&v"(f.b[0][2]), "=&v"(f.a[3]), "=&v"(f.b[0][3])
        : "v"(wa), "v"(xa));
}

template <>
__device__ __forceinline__ void lds_stage<2, 4>(StageFrags<2, 4>& f, uint32_t wa, uint32_t xa)
{
    asm volatile(
        "ds_read_b128 %0, %12 offset:0\n"
        "ds_read_b128 %1, %13 offset:0\n"
        "ds_read_b128 %2, %13 offset:16384\n"
        "ds_read_b128 %3, %12 offset:1024\n"
        "ds_read_b128 %4, %13 offset:1024\n"
        "ds_read_b128 %5, %13 offset:17408\n"
        "ds_read_b128 %6, %12 offset:2048\n"
        "ds_read_b128 %7, %13 offset:2048\n"
        "ds_read_b128 %8, %13 offset:18432\n"
        "ds_read_b128 %9, %12 offset:3072\n"
        "ds_read_b128 %10, %13 offset:3072\n"
        "ds_read_b128 %11, %13 offset:19456\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f.a[0]), "=&v"(f.b[0][0]), "=&v"(f.b[1][0]), "=&v"(f.a[1]),
          "=&v"(f.b[0][1]), "=&v"(f.b[1][1]), "=&v"(f.a[2]), "=&v"(f.b[0][2]),
          "=&v"(f.b[1][2]), "=&v"(f.a[3]), "=&v"(f.b[0][3]), "=&v"(f.b[1][3])
        : "v"(wa), "v"(xa));
}

template <>
__device__ __forceinline__ void lds_stage<3, 4>(StageFrags<3, 4>& f, uint32_t wa, uint32_t xa)
{
    asm volatile(
        "ds_read_b128 %0, %16 offset:0\n"
        "ds_read_b128 %1, %17 offset:0\n"
        "ds_read_b128 %2, %17 offset:16384\n"
        "ds_read_b128 %3, %17 offset:32768\n"
        "ds_read_b128 %4, %16 offset:1024\n"
        "ds_read_b128 %5, %17 offset:1024\n"
        "ds_read_b128 %6, %17 offset:17408\n"
        "ds_read_b128 %7, %17 offset:33792\n"
        "ds_read_b128 %8, %16 offset:2048\n"
        "ds_read_b128 %9, %17 offset:2048\n"
        "ds_read_b128 %10, %17 offset:18432\n"
        "ds_read_b128 %11, %17 offset:34816\n"
        "ds_read_b128 %12, %16 offset:3072\n"
        "ds_read_b128 %13, %17 offset:3072\n"
        "ds_read_b128 %14, %17 offset:19456\n"
        "ds_read_b128 %15, %17 offset:35840\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f.a[0]), "=&v"(f.b[0][0]), "=&v"(f.b[1][0]), "=&v"(f.b[2][0]),
          "=&v"(f.a[1]), "=&v"(f.b[0][1]), "=&v"(f.b[1][1]), "=&v"(f.b[2][1]),
          "=&v"(f.a[2]), "=&v"(f.b[0][2]), "=&v"(f.b[1][2]), "=&v"(f.b[2][2]),
          "=&v"(f.a[3]), "=&v"(f.b[0][3]), "=&v"(f.b[1][3]), "=&v"(f.b[2][3])
        : "v"(wa), "v"(xa));
}

template <>
__device__ __forceinline__ void lds_stage<4, 4>(StageFrags<4, 4>& f, uint32_t wa, uint32_t xa)
{
    asm volatile(
        "ds_read_b128 %0, %20 offset:0\n"
        "ds_read_b128 %1, %21 offset:0\n"
        "ds_read_b128 %2, %21 offset:16384\n"
        "ds_read_b128 %3, %21 offset:32768\n"
        "ds_read_b128 %4, %21 offset:49152\n"
        "ds_read_b128 %5, %20 offset:1024\n"
        "ds_read_b128 %6, %21 offset:1024\n"
        "ds_read_b128 %7, %21 offset:17408\n"
        "ds_read_b128 %8, %21 offset:33792\n"
        "ds_read_b128 %9, %21 offset:50176\n"
        "ds_read_b128 %10, %20 offset:2048\n"
        "ds_read_b128 %11, %21 offset:2048\n"
        "ds_read_b128 %12, %21 offset:18432\n"
        "ds_read_b128 %13, %21 offset:34816\n"
        "ds_read_b128 %14, %21 offset:51200\n"
        "ds_read_b128 %15, %20 offset:3072\n"
        "ds_read_b128 %16, %21 offset:3072\n"
        "ds_read_b128 %17, %21 offset:19456\n"
        "ds_read_b128 %18, %21 offset:35840\n"
        "ds_read_b128 %19, %21 offset:52224\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f.a[0]), "=&v"(f.b[0][0]), "=&v"(f.b[1][0]), "=&v"(f.b[2][0]),
          "=&v"(f.b[3][0]), "=&v"(f.a[1]), "=&v"(f.b[0][1]), "=&v"(f.b[1][1]),
          "=&v"(f.b[2][1]), "=&v"(f.b[3][1]), "=&v"(f.a[2]), "=&v"(f.b[0][2]),
          "=&v"(f.b[1][2]), "=&v"(f.b[2][2]), "=&v"(f.b[3][2]), "=&v"(f.a[3]),
          "=&v"(f.b[0][3]), "=&v"(f.b[1][3]), "=&v"(f.b[2][3]), "=&v"(f.b[3][3])
        : "v"(wa), "v"(xa));
}

// ---------------------------------------------------------------------------
// Token-resident weight stream.  A work item is (pair, K split, projection,
// 64-row tile); items that share a pair and split share the token slice
// [16 TB tokens][one split of K], which sits in LDS (as MFMA B fragments) for as
// long as a workgroup works on that slice.  Each workgroup takes a run of items
// inside one slice, so it loads its slice once.  The weights need no sharing:
// each wave streams its own 16 rows through a private ring of NS LDS slots by
// DMA and waits only on its own vector-memory counter, so the waves meet at a
// barrier only once, after the slice has landed.
// Every slot also carries the 16 rows' scales (one 4-byte DMA).  An item ends
// with the epilogue, or (S.partials) stores its int32 partial tile, which the
// following quantisation launch sums over the splits (rebuild mode).
struct XresItem {
    int pair, split, proj, local;
};

__device__ __forceinline__ XresItem xres_item(const StackStep& S, int item)
{
    const int per_split = S.tile_off[S.nproj];
    const int per_pair = per_split * S.splits;
    XresItem it;
    it.pair = item / per_pair;
    int r = item - it.pair * per_pair;
    it.split = r / per_split;
    r -= it.split * per_split;
    int j = 0;
#pragma unroll
    for (int q = 1; q < 6; ++q)
        if (q < S.nproj && r >= S.tile_off[q]) j = q;
    it.proj = j;
    it.local = r - S.tile_off[j];
    return it;
}

// 128 tokens (eight blocks of 16) with token slices of 8 k-blocks: token block tb
// at xa + (8 tb + i) KB.  Two assembly blocks of two k-blocks each, each ending
// with its own wait, so no operand is used before it has landed.
template <>
__device__ __forceinline__ void lds_stage<8, 4>(StageFrags<8, 4>& f, uint32_t wa, uint32_t xa)
{
#define PF_XR8_HALF(I0, I1, A, XB)                                                       \
    asm volatile(                                                                        \
        "ds_read_b128 %0, %18 offset:" #A "\n"                                           \
        "ds_read_b128 %1, %19 offset:" #XB "\n"                                          \
        "ds_read_b128 %2, %19 offset:8192+" #XB "\n"                                     \
        "ds_read_b128 %3, %19 offset:16384+" #XB "\n"                                    \
        "ds_read_b128 %4, %19 offset:24576+" #XB "\n"                                    \
        "ds_read_b128 %5, %19 offset:32768+" #XB "\n"                                    \
        "ds_read_b128 %6, %19 offset:40960+" #XB "\n"                                    \
        "ds_read_b128 %7, %19 offset:49152+" #XB "\n"                                    \
        "ds_read_b128 %8, %19 offset:57344+" #XB "\n"                                    \
        "ds_read_b128 %9, %18 offset:1024+" #A "\n"                                      \
        "ds_read_b128 %10, %19 offset:1024+" #XB "\n"                                    \
        "ds_read_b128 %11, %19 offset:9216+" #XB "\n"                                    \
        "ds_read_b128 %12, %19 offset:17408+" #XB "\n"                                   \
        "ds_read_b128 %13, %19 offset:25600+" #XB "\n"                                   \
        "ds_read_b128 %14, %19 offset:33792+" #XB "\n"                                   \
        "ds_read_b128 %15, %19 offset:41984+" #XB "\n"                                   \
        "ds_read_b128 %16, %19 offset:50176+" #XB "\n"                                   \
        "ds_read_b128 %17, %19 offset:58368+" #XB "\n"                                   \
        "s_waitcnt lgkmcnt(0)"                                                           \
        : "=&v"(f.a[I0]), "=&v"(f.b[0][I0]), "=&v"(f.b[1][I0]), "=&v"(f.b[2][I0]),       \
          "=&v"(f.b[3][I0]), "=&v"(f.b[4][I0]), "=&v"(f.b[5][I0]), "=&v"(f.b[6][I0]),    \
          "=&v"(f.b[7][I0]), "=&v"(f.a[I1]), "=&v"(f.b[0][I1]), "=&v"(f.b[1][I1]),       \
          "=&v"(f.b[2][I1]), "=&v"(f.b[3][I1]), "=&v"(f.b[4][I1]), "=&v"(f.b[5][I1]),    \
          "=&v"(f.b[6][I1]), "=&v"(f.b[7][I1])                                           \
        : "v"(wa), "v"(xa))
    PF_XR8_HALF(0, 1, 0, 0);
    PF_XR8_HALF(2, 3, 2048, 2048);
#undef PF_XR8_HALF
}

template <int TB, int KP, int NS>
__global__ __launch_bounds__(256) void k_gemm_xres(StackStep S, int wg_per_group, int per_wg)
{
    constexpr int kKsMax = TB <= 4 ? 16 : 8;            // k-blocks per split, at most
    constexpr int kXBytes = TB * kKsMax * 1024;         // resident token slice
    constexpr int kXPerWave = TB * kKsMax / 4;          // token DMAs per wave per slice
    constexpr int kSlot = KP * 1024 + 256;              // KP k-blocks of 16 rows + 64 scales
    constexpr int kLw = KP + 1;                         // DMAs per wave per stage
    static_assert(kLw * (NS - 1) <= 63, "vmcnt range");
    static_assert(KP == 2 || KP == 4, "lds_stage reads 2 or 4 k-blocks");
    constexpr int kXsBytes = TB <= 4 ? 256 : 512;       // token scales: 64 or 128
    __shared__ __attribute__((aligned(16))) int8_t xl[kXBytes + kXsBytes];
    __shared__ __attribute__((aligned(16))) int8_t ring[4][NS * kSlot];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // workgroup -> a run of items inside one (pair, split) group, so the token
    // slice is loaded once
    const int per_group = S.tile_off[S.nproj];
    const int grp = (int)blockIdx.x / wg_per_group, j = (int)blockIdx.x % wg_per_group;
    const int i0 = grp * per_group + j * per_wg;
    const int i1 = min(i0 + per_wg, (grp + 1) * per_group);
    if (i0 >= i1) return;
    const int nkb = S.K >> 6;
    const int ksb = S.kb_per_split;                     // <= kKsMax
    const int ppi = (ksb + KP - 1) / KP;                // stages per item
    const int total = (i1 - i0) * ppi;
    // Copies take a fragment as 16 rows x 64 bytes with lane l on row l / 4,
    // so that four consecutive lanes read one row's 64 contiguous bytes (the
    // address unit serves that ~2.5x faster than one 16-byte piece of each of
    // 16 rows per lane group).  Lane l fetches row r = l / 4, piece
    // (l % 4) ^ ((r / 2) % 4), and lands at 16 l: piece c of row r sits at
    // 64 r + 16 (c ^ ((r / 2) % 4)).  The MFMA operand of lane l (row l % 16,
    // piece l / 16) is then at `lofs`, and the reads of 8 consecutive lanes hit
    // 8 different 16-byte bank groups.
    const int crow = lane >> 2;                         // row (or token) this lane copies
    const int koff = ((lane & 3) ^ ((lane >> 3) & 3)) << 4;
    const uint32_t lofs = (uint32_t)((lane & 15) * 64 + (((lane >> 4) ^ ((lane >> 1) & 3)) << 4));
    int8_t* myring = ring[wave];

    // ---- token slice of (pair, split) into LDS: fragment (tb, i) at (tb*kKsMax + i) KB
    auto xload = [&](const XresItem& it) {
        const StepPair& pp = S.pair[it.pair];
        const int kb0 = it.split * ksb;
        const int kbl = min(kb0 + ksb, nkb) - 1;        // last valid k-block of the split
#pragma unroll
        for (int u = 0; u < kXPerWave; ++u) {
            const int q = wave + 4 * u, tb = q / kKsMax, i = q % kKsMax;
            const int tok = tb * 16 + crow;
            const int kb = min(kb0 + i, kbl);
            dma16(pp.X + (int64_t)(tok < pp.M ? tok : 0) * S.ldx + (int64_t)kb * 64 + koff,
                  xl + q * 1024);
        }
        if (wave == 0) dma4(pp.xs + min(lane, pp.M - 1), xl + kXBytes);
        if (TB > 4 && wave == 1) dma4(pp.xs + min(64 + lane, pp.M - 1), xl + kXBytes + 256);
    };

    // ---- issue side: this wave's weight rows of the item being loaded
    int icur = -1;
    const int8_t* iw = nullptr;
    const float* isc = nullptr;
    int ikb0 = 0, ikbl = 0;
    auto issue = [&](int g) {
        if (g >= total) return;
        const int item = i0 + g / ppi, piece = g - (g / ppi) * ppi;
        if (item != icur) {
            icur = item;
            const XresItem it = xres_item(S, item);
            const StepPair& pp = S.pair[it.pair];
            const int N = S.rows[it.proj];
            const int row0 = it.local * 64 + wave * 16;
            iw = pp.W[it.proj] + (int64_t)min(row0 + crow, N - 1) * S.K + koff;
            isc = pp.ws[it.proj] + min(row0 + (lane & 15), N - 1);    // scale l at 4 l
            ikb0 = it.split * ksb;
            ikbl = min(ikb0 + ksb, nkb) - 1;
        }
        int8_t* slot = myring + (g % NS) * kSlot;
#pragma unroll
        for (int i = 0; i < KP; ++i)
            dma16(iw + (int64_t)min(ikb0 + piece * KP + i, ikbl) * 64, slot + i * 1024);
        dma4(isc, slot + KP * 1024);
    };

    v4i acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = v4i{0, 0, 0, 0};

    // token slice first, then the first NS - 1 weight stages; loads complete in
    // issue order, so waiting until only the weight stages are outstanding
    // leaves them in flight while the slice is made visible to every wave
    XresItem cur = xres_item(S, i0);
    xload(cur);
#pragma unroll
    for (int g = 0; g < NS - 1; ++g) issue(g);
    if (total >= NS - 1) wait_vmcnt<(NS - 1) * kLw>();
    else wait_vmcnt<0>();
    stage_barrier();

    for (int g = 0; g < total; ++g) {
        const int item = i0 + g / ppi, piece = g - (g / ppi) * ppi;
        if (piece == 0 && g > 0) cur = xres_item(S, item);   // same (pair, split) throughout
        const int ahead = min(NS - 2, total - 1 - g);
        if (ahead <= 0) wait_vmcnt<0>();
        else if (ahead == 1) wait_vmcnt<kLw>();
        else if (ahead == 2) wait_vmcnt<2 * kLw>();
        else if (ahead == 3) wait_vmcnt<3 * kLw>();
        else wait_vmcnt<4 * kLw>();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        issue(g + NS - 1);                               // reuses the slot of stage g - 1
        const uint32_t slot = lds_addr(myring + (g % NS) * kSlot);
        const int ks0 = piece * KP;
        const int npc = min(KP, min(ksb, nkb - cur.split * ksb) - ks0);
        // all KP k-blocks are read (k-blocks past the split's end hold clamped
        // copies); only the first npc enter the product
        StageFrags<TB, KP> f;
        lds_stage<TB, KP>(f, slot + lofs, lds_addr(xl) + ks0 * 1024 + lofs);
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            if (i < npc) {
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
                    acc[tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.a[i], f.b[tb][i], acc[tb], 0, 0, 0);
            }
        }
        if (piece == ppi - 1) {
            const StepPair& pp = S.pair[cur.pair];
            const int N = S.rows[cur.proj];
            const int nw = cur.local * 64 + wave * 16;
            const int rl = (lane >> 4) << 2;             // row of acc[.][0] within the wave's 16
            v4f wsl = v4f{0.f, 0.f, 0.f, 0.f};
            if (!S.partials) wsl = lds_read_v4f(slot + KP * 1024 + rl * 4);   // rows rl .. rl + 3
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int tok = tb * 16 + (lane & 15);
                const int n = nw + rl;                   // first of this lane's 4 rows
                if (tok < pp.M) {
                    if (!S.partials) {
                        const float xs = lds_read_f32(lds_addr(xl + kXBytes) + tok * 4);
                        float4 v;
                        v.x = epilogue(acc[tb][0], wsl[0], xs);
                        v.y = epilogue(acc[tb][1], wsl[1], xs);
                        v.z = epilogue(acc[tb][2], wsl[2], xs);
                        v.w = epilogue(acc[tb][3], wsl[3], xs);
                        if (!((S.nostore >> cur.proj) & 1u)) {
                            float* y = pp.Y + S.yoff[cur.proj] + (int64_t)tok * S.ldy + n;
                            if (n + 3 < N) {
                                *reinterpret_cast<float4*>(y) = v;   // rows n..n+3: 16 bytes
                            } else {
                                if (n < N) y[0] = v.x;
                                if (n + 1 < N) y[1] = v.y;
                                if (n + 2 < N) y[2] = v.z;
                            }
                        }
                        float* kvr = step_kv(S, pp, cur.proj);
                        if (pp.Y2 || kvr) {
                            float* y2 = kvr ? kvr + (int64_t)tok * S.ldkv + n : pp.Y2 + (int64_t)tok * S.ldy2 + n;
                            if (n < N) y2[0] = v.x;
                            if (n + 1 < N) y2[1] = v.y;
                            if (n + 2 < N) y2[2] = v.z;
                            if (n + 3 < N) y2[3] = v.w;
                        }
                    } else {
                        int* part = pp.part + (int64_t)cur.split * S.part_stride + (int64_t)tok * S.ldp + n;
                        if (n + 3 < N) {
                            *reinterpret_cast<v4i*>(part) = acc[tb];
                        } else {
#pragma unroll
                            for (int r = 0; r < 3; ++r)
                                if (n + r < N) part[r] = acc[tb][r];
                        }
                    }
                }
                acc[tb] = v4i{0, 0, 0, 0};
            }
        }
    }
}

// Up to 32 tokens (TB <= 2) the LDS of a workgroup (token slice + four rings of
// five 2-k-block stages, 79 KB at TB = 2) fits twice on a compute unit: the
// grid targets two workgroups per CU, so while one of them waits for its first
// data the other streams, and launches of other streams find room.  Larger
// token slices take 4-k-block stages at one workgroup per CU; 65 to 128 tokens
// run as eight blocks with slices of at most 8 k-blocks (64 KB).  Each workgroup
// takes a run of tiles inside one (pair, split) slice.
hipError_t launch_gemm_xres(const StackStep& S, int token_blocks, hipStream_t s)
{
    const int groups = S.npairs * S.splits;              // (pair, split) token slices
    const int per_group = S.tile_off[S.nproj];           // tiles per slice
    if (groups <= 0 || per_group <= 0) return hipSuccess;
    if (token_blocks > 4 && token_blocks <= 8) token_blocks = 8;   // 65..128 tokens: eight blocks
    if (S.kb_per_split > xres_max_kb(token_blocks) || (S.splits > 1 && !S.partials)) return hipErrorInvalidValue;
    const int target = token_blocks <= 2 ? 2 * kComputeUnits : kComputeUnits;
    int wpg = target / groups;
    if (wpg < 1) wpg = 1;
    if (wpg > per_group) wpg = per_group;
    const int per_wg = (per_group + wpg - 1) / wpg;
    const dim3 g(groups * wpg), b(256);
    switch (token_blocks) {
        case 1: PF_LAUNCH((k_gemm_xres<1, 2, 5>), g, b, 0, s, S, wpg, per_wg); break;
        case 2: PF_LAUNCH((k_gemm_xres<2, 2, 5>), g, b, 0, s, S, wpg, per_wg); break;
        case 3: PF_LAUNCH((k_gemm_xres<3, 4, 4>), g, b, 0, s, S, wpg, per_wg); break;
        case 4: PF_LAUNCH((k_gemm_xres<4, 4, 4>), g, b, 0, s, S, wpg, per_wg); break;
        case 8: PF_LAUNCH((k_gemm_xres<8, 4, 4>), g, b, 0, s, S, wpg, per_wg); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pf
