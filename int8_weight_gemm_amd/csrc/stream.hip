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
        case 1: hipLaunchKernelGGL((k_gemm_stream<1, 4, 4>), g, b, 0, s, S, ntiles); break;
        case 2: hipLaunchKernelGGL((k_gemm_stream<2, 4, 3>), g, b, 0, s, S, ntiles); break;
        case 3: hipLaunchKernelGGL((k_gemm_stream<3, 4, 3>), g, b, 0, s, S, ntiles); break;
        case 4: hipLaunchKernelGGL((k_gemm_stream<4, 4, 3>), g, b, 0, s, S, ntiles); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pf
