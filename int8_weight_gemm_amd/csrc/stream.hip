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
#include "problems.hpp"

namespace pf {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

__device__ __forceinline__ void dma16(const int8_t* g, int8_t* lds_base)
{
    __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}

__device__ __forceinline__ void dma4(const float* g, int8_t* lds_base)
{
    __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_base, 4, 0, 0);
}

// s_waitcnt with only the vector-memory counter limited to N (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads (which would wait
// for every outstanding load, draining the DMA pipeline).  Completion of this
// wave's DMAs is established by wait_vmcnt before it; the signal fences keep
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void stage_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

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
    const int koff = (lane >> 4) << 4;

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
            const int n = min(local * 64 + wave * 16 + (lane & 15), P.N - 1);
            iw = P.W + (int64_t)n * P.K + koff;
#pragma unroll
            for (int u = 0; u < kXPerWave; ++u) {
                const int q = wave + 4 * u, tb = q / KP;
                const int tok = tb * 16 + (lane & 15);
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
                const v4i a = *reinterpret_cast<const v4i*>(base + (wave * KP + i) * 1024 + lane * 16);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const v4i b = *reinterpret_cast<const v4i*>(base + kWBytes + (tb * KP + i) * 1024 + lane * 16);
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

// ---------------------------------------------------------------------------
// Token-resident weight stream.  A work item is (pair, K split, projection,
// 64-row tile); items that share a pair and split share the token slice
// [16 TB tokens][one split of K], which sits in LDS (as MFMA B fragments) for as
// long as a workgroup works on that slice.  Each workgroup takes a contiguous
// run of items, so it loads a slice once per run, not once per tile.  The
// weights need no sharing: each wave streams its own 16 rows through a private
// ring of NS LDS slots by DMA and waits only on its own vector-memory counter,
// so the waves never meet at a barrier except when the token slice changes.
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

template <int TB, int KP, int NS>
__global__ __launch_bounds__(256) void k_gemm_xres(StackStep S, int nitems, int per_wg)
{
    constexpr int kKsMax = 16;                          // k-blocks per split, at most
    constexpr int kXBytes = TB * kKsMax * 1024;         // resident token slice
    constexpr int kXPerWave = TB * kKsMax / 4;          // token DMAs per wave per slice
    constexpr int kSlot = KP * 1024 + 256;              // KP k-blocks of 16 rows + 64 scales
    constexpr int kLw = KP + 1;                         // DMAs per wave per stage
    static_assert(kLw * (NS - 2) <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(16))) int8_t xl[kXBytes + 256];
    __shared__ __attribute__((aligned(16))) int8_t ring[4][NS * kSlot];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i0 = (int)blockIdx.x * per_wg;
    const int i1 = min(i0 + per_wg, nitems);
    if (i0 >= i1) return;
    const int nkb = S.K >> 6;
    const int ksb = S.kb_per_split;                     // <= kKsMax
    const int ppi = (ksb + KP - 1) / KP;                // stages per item
    const int total = (i1 - i0) * ppi;
    const int koff = (lane >> 4) << 4;
    int8_t* myring = ring[wave];

    // ---- token slice of (pair, split) into LDS: fragment (tb, i) at (tb*kKsMax + i) KB
    auto xload = [&](const XresItem& it) {
        const StepPair& pp = S.pair[it.pair];
        const int kb0 = it.split * ksb;
        const int kbl = min(kb0 + ksb, nkb) - 1;        // last valid k-block of the split
#pragma unroll
        for (int u = 0; u < kXPerWave; ++u) {
            const int q = wave + 4 * u, tb = q / kKsMax, i = q % kKsMax;
            const int tok = tb * 16 + (lane & 15);
            const int kb = min(kb0 + i, kbl);
            dma16(pp.X + (int64_t)(tok < pp.M ? tok : 0) * S.ldx + (int64_t)kb * 64 + koff,
                  xl + q * 1024);
        }
        if (wave == 0) dma4(pp.xs + min(lane, pp.M - 1), xl + kXBytes);
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
            iw = pp.W[it.proj] + (int64_t)min(row0 + (lane & 15), N - 1) * S.K + koff;
            isc = pp.ws[it.proj] + min(row0 + (lane & 15), N - 1);
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

    XresItem cur = xres_item(S, i0);
    xload(cur);
    wait_vmcnt<0>();
    stage_barrier();
#pragma unroll
    for (int g = 0; g < NS - 1; ++g) issue(g);

    for (int g = 0; g < total; ++g) {
        const int item = i0 + g / ppi, piece = g - (g / ppi) * ppi;
        if (piece == 0 && g > 0) {
            const XresItem nx = xres_item(S, item);
            if (nx.pair != cur.pair || nx.split != cur.split) {
                stage_barrier();                         // every wave is done with the old slice
                xload(nx);
                wait_vmcnt<0>();
                stage_barrier();
            }
            cur = nx;
        }
        const int ahead = min(NS - 2, total - 1 - g);
        if (ahead <= 0) wait_vmcnt<0>();
        else if (ahead == 1) wait_vmcnt<kLw>();
        else if (ahead == 2) wait_vmcnt<2 * kLw>();
        else if (ahead == 3) wait_vmcnt<3 * kLw>();
        else wait_vmcnt<4 * kLw>();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        issue(g + NS - 1);                               // reuses the slot of stage g - 1
        const int8_t* slot = myring + (g % NS) * kSlot;
        const int ks0 = piece * KP;
        const int npc = min(KP, min(ksb, nkb - cur.split * ksb) - ks0);
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            if (i < npc) {
                const v4i a = *reinterpret_cast<const v4i*>(slot + i * 1024 + lane * 16);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const v4i b = *reinterpret_cast<const v4i*>(xl + (tb * kKsMax + ks0 + i) * 1024 + lane * 16);
                    acc[tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[tb], 0, 0, 0);
                }
            }
        }
        if (piece == ppi - 1) {
            const StepPair& pp = S.pair[cur.pair];
            const int N = S.rows[cur.proj];
            const int nw = cur.local * 64 + wave * 16;
            const int rl = (lane >> 4) << 2;             // row of acc[.][0] within the wave's 16
            const float* wsl = reinterpret_cast<const float*>(slot + KP * 1024);
            const float* xsl = reinterpret_cast<const float*>(xl + kXBytes);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int tok = tb * 16 + (lane & 15);
                const int n = nw + rl;                   // first of this lane's 4 rows
                if (tok < pp.M) {
                    if (!S.partials) {
                        const float xs = xsl[tok];
                        float4 v;
                        v.x = epilogue(acc[tb][0], wsl[rl], xs);
                        v.y = epilogue(acc[tb][1], wsl[rl + 1], xs);
                        v.z = epilogue(acc[tb][2], wsl[rl + 2], xs);
                        v.w = epilogue(acc[tb][3], wsl[rl + 3], xs);
                        float* y = pp.Y + S.yoff[cur.proj] + (int64_t)tok * S.ldy + n;
                        if (n + 3 < N) {
                            *reinterpret_cast<float4*>(y) = v;   // rows n..n+3: 16 bytes
                        } else {
                            if (n < N) y[0] = v.x;
                            if (n + 1 < N) y[1] = v.y;
                            if (n + 2 < N) y[2] = v.z;
                        }
                        if (pp.Y2) {
                            float* y2 = pp.Y2 + (int64_t)tok * S.ldy2 + n;
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

// One workgroup per compute unit (the LDS holds a token slice and four rings),
// each taking a contiguous run of work items.
hipError_t launch_gemm_xres(const StackStep& S, int token_blocks, hipStream_t s)
{
    const int nitems = S.npairs * S.splits * S.tile_off[S.nproj];
    if (nitems <= 0) return hipSuccess;
    if (S.kb_per_split > 16 || (S.splits > 1 && !S.partials)) return hipErrorInvalidValue;
    const int grid = nitems < 256 ? nitems : 256;
    const int per_wg = (nitems + grid - 1) / grid;
    const dim3 g((nitems + per_wg - 1) / per_wg), b(256);
    switch (token_blocks) {
        case 1: PF_LAUNCH((k_gemm_xres<1, 4, 6>), g, b, 0, s, S, nitems, per_wg); break;
        case 2: PF_LAUNCH((k_gemm_xres<2, 4, 6>), g, b, 0, s, S, nitems, per_wg); break;
        case 3: PF_LAUNCH((k_gemm_xres<3, 4, 4>), g, b, 0, s, S, nitems, per_wg); break;
        case 4: PF_LAUNCH((k_gemm_xres<4, 4, 4>), g, b, 0, s, S, nitems, per_wg); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pf
