// tiled.hip — the int8 product for chunks of more than 64 tokens (gfx950).
//
// "Batched Prefill" (cellm), §The arithmetic: with hundreds of tokens per chunk
// every weight byte feeds hundreds of multiply-adds, so the product is bound by
// the matrix cores, not by HBM.  The kernel is laid out for v_mfma_i32_16x16x64_i8
// at full rate:
//  * a workgroup owns 256 weight rows x 32 WM tokens (WM = 8 or 4); each of its
//    four waves owns 128 rows x 16 WM tokens, i.e. 8 x WM accumulator blocks of
//    16 x 16 (256 or 128 accumulation registers), so each operand fragment read
//    from LDS feeds WM or 8 MFMAs;
//  * a stage is one k-block (64 bytes of K) of the tile's 256 weight rows and
//    32 WM tokens, copied by global_load_lds_dwordx4 straight into LDS in MFMA
//    operand order (fragment = 16 rows x 64 bytes, lane l's 16 bytes at 16 l);
//    NS stages are in flight, one barrier per stage;
//  * the fragments of stage g + 1 are read from LDS while the MFMAs of stage g
//    run (two register sets);
//  * workgroups on one XCD (blockIdx % 8) take consecutive tiles, and the token
//    tiles of one band of weight rows are consecutive, so the band is fetched
//    from HBM once into that XCD's L2 and shared.
// Epilogue: y[t][n] = fl(fl(acc) * fl(ws[n] * xs[t])), 16-byte stores of four
// consecutive rows of one token where alignment allows.
#include "device.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"
#include "problems.hpp"

namespace pf {

constexpr int kTlWN = 8;                     // 16-row blocks per wave (128 rows)

// One stage's operand fragments of a wave: 8 weight fragments, WM token ones.
template <int WM>
struct TlFrags {
    v4i a[kTlWN];
    v4i b[WM];
};

// Issue the wave's LDS reads of one stage (weight fragments at a + 1 KB i,
// token fragments at b + 1 KB j) without waiting; tl_wait waits for them.  The
// wait names every destination register, so no use of one can be placed
// before it.
template <int WM>
__device__ __forceinline__ void tl_issue(TlFrags<WM>& f, uint32_t a, uint32_t b);
template <int WM>
__device__ __forceinline__ void tl_wait(TlFrags<WM>& f);

template <>
__device__ __forceinline__ void tl_issue<8>(TlFrags<8>& f, uint32_t a, uint32_t b)
{
    asm volatile(
        "ds_read_b128 %0, %16 offset:0\n"
        "ds_read_b128 %1, %16 offset:1024\n"
        "ds_read_b128 %2, %16 offset:2048\n"
        "ds_read_b128 %3, %16 offset:3072\n"
        "ds_read_b128 %4, %16 offset:4096\n"
        "ds_read_b128 %5, %16 offset:5120\n"
        "ds_read_b128 %6, %16 offset:6144\n"
        "ds_read_b128 %7, %16 offset:7168\n"
        "ds_read_b128 %8, %17 offset:0\n"
        "ds_read_b128 %9, %17 offset:1024\n"
        "ds_read_b128 %10, %17 offset:2048\n"
        "ds_read_b128 %11, %17 offset:3072\n"
        "ds_read_b128 %12, %17 offset:4096\n"
        "ds_read_b128 %13, %17 offset:5120\n"
        "ds_read_b128 %14, %17 offset:6144\n"
        "ds_read_b128 %15, %17 offset:7168\n"
        : "=&v"(f.a[0]), "=&v"(f.a[1]), "=&v"(f.a[2]), "=&v"(f.a[3]),
          "=&v"(f.a[4]), "=&v"(f.a[5]), "=&v"(f.a[6]), "=&v"(f.a[7]),
          "=&v"(f.b[0]), "=&v"(f.b[1]), "=&v"(f.b[2]), "=&v"(f.b[3]),
          "=&v"(f.b[4]), "=&v"(f.b[5]), "=&v"(f.b[6]), "=&v"(f.b[7])
        : "v"(a), "v"(b));
}

template <>
__device__ __forceinline__ void tl_wait<8>(TlFrags<8>& f)
{
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]),
                 "+v"(f.a[4]), "+v"(f.a[5]), "+v"(f.a[6]), "+v"(f.a[7]),
                 "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3]),
                 "+v"(f.b[4]), "+v"(f.b[5]), "+v"(f.b[6]), "+v"(f.b[7]));
}

template <>
__device__ __forceinline__ void tl_issue<4>(TlFrags<4>& f, uint32_t a, uint32_t b)
{
    asm volatile(
        "ds_read_b128 %0, %12 offset:0\n"
        "ds_read_b128 %1, %12 offset:1024\n"
        "ds_read_b128 %2, %12 offset:2048\n"
        "ds_read_b128 %3, %12 offset:3072\n"
        "ds_read_b128 %4, %12 offset:4096\n"
        "ds_read_b128 %5, %12 offset:5120\n"
        "ds_read_b128 %6, %12 offset:6144\n"
        "ds_read_b128 %7, %12 offset:7168\n"
        "ds_read_b128 %8, %13 offset:0\n"
        "ds_read_b128 %9, %13 offset:1024\n"
        "ds_read_b128 %10, %13 offset:2048\n"
        "ds_read_b128 %11, %13 offset:3072\n"
        : "=&v"(f.a[0]), "=&v"(f.a[1]), "=&v"(f.a[2]), "=&v"(f.a[3]),
          "=&v"(f.a[4]), "=&v"(f.a[5]), "=&v"(f.a[6]), "=&v"(f.a[7]),
          "=&v"(f.b[0]), "=&v"(f.b[1]), "=&v"(f.b[2]), "=&v"(f.b[3])
        : "v"(a), "v"(b));
}

template <>
__device__ __forceinline__ void tl_wait<4>(TlFrags<4>& f)
{
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]),
                 "+v"(f.a[4]), "+v"(f.a[5]), "+v"(f.a[6]), "+v"(f.a[7]),
                 "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3]));
}

// vmcnt limited to `stages` whole stages of kL DMAs (stages <= NS - 1 <= 7).
template <int kL>
__device__ __forceinline__ void wait_stages(int stages)
{
    switch (stages) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<kL>(); break;
        case 2: wait_vmcnt<(2 * kL > 63 ? 63 : 2 * kL)>(); break;
        case 3: wait_vmcnt<(3 * kL > 63 ? 63 : 3 * kL)>(); break;
        case 4: wait_vmcnt<(4 * kL > 63 ? 63 : 4 * kL)>(); break;
        default: wait_vmcnt<(5 * kL > 63 ? 63 : 5 * kL)>(); break;
    }
}

// One 256 x 32 WM output tile of problem P (tile index `local`, token tiles
// fastest).
template <int WM, int NS>
__device__ __forceinline__ void tiled_block(const GemmProb& P, int local)
{
    constexpr int kFa = 2 * kTlWN, kFb = 2 * WM;          // fragments per stage
    constexpr int kStage = (kFa + kFb) * 1024;
    constexpr int kL = (kFa + kFb) / 4;                   // DMAs per wave per stage
    static_assert((kFa + kFb) % 4 == 0, "fragments must split evenly over the waves");
    static_assert(kL * (NS - 1) <= 63 && NS <= 6, "vmcnt range");
    __shared__ __attribute__((aligned(16))) int8_t ring[NS * kStage];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tm = local % P.tiles_m, tn = local / P.tiles_m;
    const int n0 = tn * 32 * kTlWN, t0 = tm * 32 * WM;
    const int nkb = P.K >> 6;
    const int koff = (lane >> 4) << 4;

    // this wave copies fragments wave, wave + 4, ...: weight rows, then tokens
    // (rows and tokens past the end repeat the last one; their results are
    // never stored)
    const int8_t* src[kL];
#pragma unroll
    for (int u = 0; u < kL; ++u) {
        const int f = wave + 4 * u;
        if (f < kFa) {
            const int n = min(n0 + 16 * f + (lane & 15), P.N - 1);
            src[u] = P.W + (int64_t)n * P.K + koff;
        } else {
            const int t = min(t0 + 16 * (f - kFa) + (lane & 15), P.M - 1);
            src[u] = P.X + (int64_t)t * P.ldx + koff;
        }
    }
    auto issue = [&](int g) {                             // stage g -> slot g % NS
        if (g >= nkb) return;
        int8_t* slot = ring + (g % NS) * kStage;
#pragma unroll
        for (int u = 0; u < kL; ++u) dma16(src[u] + (int64_t)g * 64, slot + (wave + 4 * u) * 1024);
    };

    const int wn = wave >> 1, wm = wave & 1;
    const uint32_t ra = lds_addr(ring) + wn * kTlWN * 1024 + lane * 16;
    const uint32_t rb = lds_addr(ring) + (kFa + wm * WM) * 1024 + lane * 16;

    v4i acc[kTlWN][WM];
#pragma unroll
    for (int i = 0; i < kTlWN; ++i)
#pragma unroll
        for (int j = 0; j < WM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

#pragma unroll
    for (int g = 0; g < NS; ++g) issue(g);
    wait_stages<kL>(min(nkb, NS) - 1);                   // own copies of stage 0
    stage_barrier();
    TlFrags<WM> f0, f1;
    tl_issue<WM>(f0, ra, rb);

    // stage g: its fragments are in `cur`; stage g + 1 goes to `nxt`
    auto step = [&](int g, TlFrags<WM>& cur, TlFrags<WM>& nxt) {
        tl_wait<WM>(cur);
        if (g + 1 < nkb) {
            wait_stages<kL>(min(nkb - g - 2, NS - 2));   // own copies of stage g + 1
            stage_barrier();                             // ... and every wave's; stage g read by all
            issue(g + NS);                               // refills stage g's slot
            const uint32_t so = (uint32_t)(((g + 1) % NS) * kStage);
            tl_issue<WM>(nxt, ra + so, rb + so);
        }
        __builtin_amdgcn_sched_barrier(0);               // reads go out before the MFMAs
#pragma unroll
        for (int i = 0; i < kTlWN; ++i)
#pragma unroll
            for (int j = 0; j < WM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0);
        // keep the next stage's waits behind these MFMAs (they overlap its reads)
        __builtin_amdgcn_sched_barrier(0);
    };
    int g = 0;
    for (; g + 1 < nkb; g += 2) {                        // the same registers every pass
        step(g, f0, f1);
        step(g + 1, f1, f0);
    }
    if (g < nkb) step(g, f0, f1);

    // Lane l of a 16 x 16 block holds rows 4 (l / 16) .. + 3 of token l % 16.
    const bool vec = (((uintptr_t)P.Y & 15) == 0) && ((P.ldy & 3) == 0) &&
                     (!P.Y2 || ((((uintptr_t)P.Y2 & 15) == 0) && ((P.ldy2 & 3) == 0)));
    float xs[WM];
#pragma unroll
    for (int j = 0; j < WM; ++j) xs[j] = P.xs[min(t0 + wm * 16 * WM + 16 * j + (lane & 15), P.M - 1)];
#pragma unroll
    for (int i = 0; i < kTlWN; ++i) {
        const int n = n0 + wn * 16 * kTlWN + 16 * i + ((lane >> 4) << 2);
        if (n >= P.N) continue;
        float w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = P.ws[min(n + r, P.N - 1)];
#pragma unroll
        for (int j = 0; j < WM; ++j) {
            const int t = t0 + wm * 16 * WM + 16 * j + (lane & 15);
            if (t >= P.M) continue;
            float4 v;
            v.x = epilogue(acc[i][j][0], w[0], xs[j]);
            v.y = epilogue(acc[i][j][1], w[1], xs[j]);
            v.z = epilogue(acc[i][j][2], w[2], xs[j]);
            v.w = epilogue(acc[i][j][3], w[3], xs[j]);
            float* y = P.Y + (int64_t)t * P.ldy + n;
            float* y2 = P.Y2 ? P.Y2 + (int64_t)t * P.ldy2 + n : nullptr;
            if (vec && n + 3 < P.N) {
                *reinterpret_cast<float4*>(y) = v;
                if (y2) *reinterpret_cast<float4*>(y2) = v;
            } else {
                const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < P.N) {
                        y[r] = e[r];
                        if (y2) y2[r] = e[r];
                    }
            }
        }
    }
}

// Workgroup b -> tile (b % 8) * per_xcd + b / 8: the workgroups of one XCD take
// a contiguous range of tiles.  The grid is 8 per_xcd; indices past the last
// tile return at once.
__device__ __forceinline__ int xcd_tile(int per_xcd)
{
    return ((int)blockIdx.x & 7) * per_xcd + ((int)blockIdx.x >> 3);
}

template <int WM, int NS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_tiled(GemmSet set, int per_xcd)
{
    const int j = xcd_tile(per_xcd);
    if (j >= set.total_tiles) return;
    const GemmProb P = find_prob(set, j);
    tiled_block<WM, NS>(P, j - P.tile_begin);
}

template <int WM, int NS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_tiled_step(StackStep S, int per_xcd)
{
    const int j = xcd_tile(per_xcd);
    if (j >= S.npairs * S.tile_off[S.nproj]) return;
    int local;
    const GemmProb P = step_prob(S, j, local);
    tiled_block<WM, NS>(P, local);
}

int tiled_tokens(int64_t M) { return M > 128 ? 32 * 8 : 32 * 4; }

hipError_t launch_gemm_tiled(const GemmSet& set, int64_t M, hipStream_t s)
{
    if (set.total_tiles <= 0) return hipSuccess;
    const int per_xcd = (set.total_tiles + 7) / 8;
    const dim3 g(8 * per_xcd), b(256);
    if (tiled_tokens(M) == 256) PF_LAUNCH((k_gemm_tiled<8, 4>), g, b, 0, s, set, per_xcd);
    else PF_LAUNCH((k_gemm_tiled<4, 6>), g, b, 0, s, set, per_xcd);
    return hipGetLastError();
}

hipError_t launch_gemm_tiled_step(const StackStep& S, int64_t M, hipStream_t s)
{
    const int tiles = S.npairs * S.tile_off[S.nproj];
    if (tiles <= 0) return hipSuccess;
    const int per_xcd = (tiles + 7) / 8;
    const dim3 g(8 * per_xcd), b(256);
    if (tiled_tokens(M) == 256) PF_LAUNCH((k_gemm_tiled_step<8, 4>), g, b, 0, s, S, per_xcd);
    else PF_LAUNCH((k_gemm_tiled_step<4, 6>), g, b, 0, s, S, per_xcd);
    return hipGetLastError();
}

}  // namespace pf
