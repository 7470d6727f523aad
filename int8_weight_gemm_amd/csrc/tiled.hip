// tiled.hip — the int8 product for chunks of more than 64 tokens (gfx950).
//
// "Batched Prefill" (cellm), §The arithmetic: with hundreds of tokens per chunk
// every weight byte feeds hundreds of multiply-adds, so the product is bound by
// the matrix cores, not by HBM.  The kernel is laid out for v_mfma_i32_32x32x32_i8:
//  * a workgroup of eight waves (two per SIMD) owns 256 weight rows x 64 WJ
//    tokens (WJ = 4 or 2); wave (wn, wm) of the 2 x 4 grid owns 128 rows x
//    16 WJ tokens: 4 x WJ / 2 accumulator blocks of 32 x 32;
//  * a stage is one k-block (64 bytes of K) of the tile's weight rows and
//    tokens in LDS as 1 KB fragments of 16 rows x 64 bytes.  A copy gives four
//    consecutive lanes one row's 64 contiguous bytes (lane l: row l / 4), the
//    order in which the address unit serves a fragment ~2.5x faster than one
//    16-byte piece of each of 16 rows per lane group; lane l lands at 16 l, so
//    piece c of row r sits at 64 r + 16 (c ^ ((r / 2) % 4)), and the MFMA
//    operands are read with one conflict-free ds_read_b128 each; a ring of
//    four stages, one barrier per stage, and the reads of stage g + 1 are in
//    flight while the MFMAs of stage g run;
//  * every fragment, weights and tokens, is copied by global_load_lds_dwordx4,
//    three stages ahead.  These copies, 32 KB per stage and compute unit, are
//    what holds the kernel: alone (no operand reads, no MFMAs) they take about
//    80% of its time, while the operand reads and MFMAs alone take about 73%;
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


// One stage's MFMA operands of a wave: 8 weight operands (4 row blocks x 2 k
// halves), WM token ones (WM / 2 token blocks x 2 k halves).
template <int WM>
struct TlFrags {
    v4i a[8];
    v4i b[WM];
};

// Issue the wave's LDS reads of one stage without waiting; tl_wait waits for
// them.  Operand q = 2 i + kh (32-row block i, k half kh) is read at
// a_kh + 2 KB i (weights) or b_kh + 2 KB i (tokens), a_kh and b_kh carrying
// the lane's own offset in the block for k half kh.  The wait names every
// destination register, so no use of one can be placed before it.
template <int WM>
__device__ __forceinline__ void tl_issue(TlFrags<WM>& f, uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1);
template <int WM>
__device__ __forceinline__ void tl_wait(TlFrags<WM>& f);

template <>
__device__ __forceinline__ void tl_issue<4>(TlFrags<4>& f, uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1)
{
    asm volatile(
        "ds_read_b128 %0, %12 offset:0\n"
        "ds_read_b128 %1, %13 offset:0\n"
        "ds_read_b128 %2, %12 offset:2048\n"
        "ds_read_b128 %3, %13 offset:2048\n"
        "ds_read_b128 %4, %12 offset:4096\n"
        "ds_read_b128 %5, %13 offset:4096\n"
        "ds_read_b128 %6, %12 offset:6144\n"
        "ds_read_b128 %7, %13 offset:6144\n"
        "ds_read_b128 %8, %14 offset:0\n"
        "ds_read_b128 %9, %15 offset:0\n"
        "ds_read_b128 %10, %14 offset:2048\n"
        "ds_read_b128 %11, %15 offset:2048\n"
        : "=&v"(f.a[0]), "=&v"(f.a[1]), "=&v"(f.a[2]), "=&v"(f.a[3]),
          "=&v"(f.a[4]), "=&v"(f.a[5]), "=&v"(f.a[6]), "=&v"(f.a[7]),
          "=&v"(f.b[0]), "=&v"(f.b[1]), "=&v"(f.b[2]), "=&v"(f.b[3])
        : "v"(a0), "v"(a1), "v"(b0), "v"(b1));
}

template <>
__device__ __forceinline__ void tl_issue<2>(TlFrags<2>& f, uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1)
{
    asm volatile(
        "ds_read_b128 %0, %10 offset:0\n"
        "ds_read_b128 %1, %11 offset:0\n"
        "ds_read_b128 %2, %10 offset:2048\n"
        "ds_read_b128 %3, %11 offset:2048\n"
        "ds_read_b128 %4, %10 offset:4096\n"
        "ds_read_b128 %5, %11 offset:4096\n"
        "ds_read_b128 %6, %10 offset:6144\n"
        "ds_read_b128 %7, %11 offset:6144\n"
        "ds_read_b128 %8, %12 offset:0\n"
        "ds_read_b128 %9, %13 offset:0\n"
        : "=&v"(f.a[0]), "=&v"(f.a[1]), "=&v"(f.a[2]), "=&v"(f.a[3]),
          "=&v"(f.a[4]), "=&v"(f.a[5]), "=&v"(f.a[6]), "=&v"(f.a[7]),
          "=&v"(f.b[0]), "=&v"(f.b[1])
        : "v"(a0), "v"(a1), "v"(b0), "v"(b1));
}

template <>
__device__ __forceinline__ void tl_wait<2>(TlFrags<2>& f)
{
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]),
                 "+v"(f.a[4]), "+v"(f.a[5]), "+v"(f.a[6]), "+v"(f.a[7]),
                 "+v"(f.b[0]), "+v"(f.b[1]));
}

template <>
__device__ __forceinline__ void tl_wait<4>(TlFrags<4>& f)
{
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]),
                 "+v"(f.a[4]), "+v"(f.a[5]), "+v"(f.a[6]), "+v"(f.a[7]),
                 "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3]));
}

template <>
__device__ __forceinline__ void tl_issue<8>(TlFrags<8>& f, uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1)
{
    asm volatile(
        "ds_read_b128 %0, %16 offset:0\n"
        "ds_read_b128 %1, %17 offset:0\n"
        "ds_read_b128 %2, %16 offset:2048\n"
        "ds_read_b128 %3, %17 offset:2048\n"
        "ds_read_b128 %4, %16 offset:4096\n"
        "ds_read_b128 %5, %17 offset:4096\n"
        "ds_read_b128 %6, %16 offset:6144\n"
        "ds_read_b128 %7, %17 offset:6144\n"
        "ds_read_b128 %8, %18 offset:0\n"
        "ds_read_b128 %9, %19 offset:0\n"
        "ds_read_b128 %10, %18 offset:2048\n"
        "ds_read_b128 %11, %19 offset:2048\n"
        "ds_read_b128 %12, %18 offset:4096\n"
        "ds_read_b128 %13, %19 offset:4096\n"
        "ds_read_b128 %14, %18 offset:6144\n"
        "ds_read_b128 %15, %19 offset:6144\n"
        : "=&v"(f.a[0]), "=&v"(f.a[1]), "=&v"(f.a[2]), "=&v"(f.a[3]),
          "=&v"(f.a[4]), "=&v"(f.a[5]), "=&v"(f.a[6]), "=&v"(f.a[7]),
          "=&v"(f.b[0]), "=&v"(f.b[1]), "=&v"(f.b[2]), "=&v"(f.b[3]),
          "=&v"(f.b[4]), "=&v"(f.b[5]), "=&v"(f.b[6]), "=&v"(f.b[7])
        : "v"(a0), "v"(a1), "v"(b0), "v"(b1));
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

// One 256 x 64 WJ output tile of problem P (tile index `local`, token tiles
// fastest), by NW waves (4: one per SIMD; 8: two per SIMD) in a 2 x NW/2 grid:
// wave (wn, wm) owns rows 128 wn .. + 127 and JB = 4 WJ / NW token blocks of
// 32 from token 32 JB wm: 4 x JB accumulator blocks of 32 x 32.  Stage s (one
// k-block) sits in ring slot s % 4: weight fragments 0 .. 15 (16 rows x 64
// bytes each), then token fragments 0 .. 4 WJ - 1; wave w copies fragments
// w + NW h of each by DMA.  Iteration g:
//   wait for stage g's fragments (read in iteration g - 1) and this wave's
//   copies of stage g + 1; barrier (stage g + 1 published, stage g read by
//   all); copy stage g + 4 into the slot of stage g; issue the reads of stage
//   g + 1; the MFMAs of stage g.
// With two waves per SIMD, the waves of the second row half copy after their
// first k half of MFMAs instead: a wave issuing copies issues no MFMA, and
// its SIMD's other wave then does.
// Every iteration issues the same copies (k-blocks past the end are clamped
// to the last one and land in free slots, never read), so every wait is a
// constant.
template <int WJ, int NW>
__device__ __forceinline__ void tiled_block(const GemmProb& P, int local, int kidx)
{
    constexpr int NS = 4;
    constexpr int WMT = NW / 2;                          // token parts of the wave grid
    constexpr int JB = 2 * WJ / WMT;                     // 32-token blocks per wave
    constexpr int WB = 2 * JB;                           // token operands per wave per stage
    constexpr int kFa = 16, kFb = 4 * WJ;                // fragments per stage
    constexpr int kStage = (kFa + kFb) * 1024;
    constexpr int ka = kFa / NW, kb = kFb / NW;          // copies per wave per stage
    constexpr int kOps = ka + kb;                        // vector-memory ops per wave per stage
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    static_assert(kb * NW == kFb && JB >= 1, "tile shape");
    static_assert(3 * kOps <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(16))) int8_t ring[NS * kStage];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tm = local % P.tiles_m, tn = local / P.tiles_m;
    const int n0 = tn * 256, t0 = tm * 64 * WJ;
    // this split's k-blocks: kb0 .. kb0 + nkb - 1 (all of K when unsplit)
    const int kb0 = kidx * P.kb_per_split;
    const int nkb = min(P.kb_per_split, (P.K >> 6) - kb0);
    // fragment f: rows (or tokens) 16 f .. + 15 of the k-block; lane l copies
    // row l / 4, piece (l % 4) ^ ((l / 8) % 4), to 16 l.  Rows and tokens past
    // the end repeat the last one; their results are never stored.
    const int lrow = lane & 31;
    const int crow = lane >> 2;                          // row this lane copies
    const int kof = ((lane & 3) ^ ((lane >> 3) & 3)) << 4;
    const int8_t* asrc[ka];
#pragma unroll
    for (int h = 0; h < ka; ++h) {
        const int f = wave + NW * h;
        asrc[h] = P.W + (int64_t)min(n0 + 16 * f + crow, P.N - 1) * P.K + kof;
    }
    const int8_t* bsrc[kb];
#pragma unroll
    for (int h = 0; h < kb; ++h) {
        const int f = wave + NW * h;
        bsrc[h] = P.X + (int64_t)min(t0 + 16 * f + crow, P.M - 1) * P.ldx + kof;
    }
    const uint32_t ring0 = lds_addr(ring);

    auto kbo = [&](int s) { return (int64_t)(kb0 + min(s, nkb - 1)) * 64; };
    // stage s into its slot: this wave's weight fragments w + NW h and token
    // fragments kFa + w + NW h, all by DMA (kOps copies)
    auto put = [&](int s) {
        int8_t* slot = ring + (s % NS) * kStage;
#pragma unroll
        for (int h = 0; h < ka; ++h) dma16(asrc[h] + kbo(s), slot + (wave + NW * h) * 1024);
#pragma unroll
        for (int h = 0; h < kb; ++h) dma16(bsrc[h] + kbo(s), slot + (kFa + wave + NW * h) * 1024);
    };

    // The 32 x 32 x 32 operand of rows 32 i .. + 31, k half kh: lane l needs
    // row r = l % 32, piece c = 2 kh + l / 32, which sits in fragment
    // 2 i + r / 16 at 64 (r % 16) + 16 (c ^ ((r % 16 / 2) % 4)); for k half 1
    // that is the half-0 offset with bit 5 flipped.  Any 8 consecutive lanes
    // read 8 different 16-byte bank groups.
    const uint32_t lofs = (uint32_t)(((lane >> 4) & 1) * 1024 + 64 * (lane & 15) +
                                     16 * ((lane >> 5) ^ ((lane >> 1) & 3)));   // k half 0; half 1: ^ 32
    const int wn = wave / WMT, wm = wave % WMT;
    const uint32_t ra0 = ring0 + wn * 8 * 1024 + lofs, ra1 = ring0 + wn * 8 * 1024 + (lofs ^ 32);
    const uint32_t rb0 = ring0 + (kFa + wm * WB) * 1024 + lofs, rb1 = ring0 + (kFa + wm * WB) * 1024 + (lofs ^ 32);
    const bool late_copy = NW == 8 && wn == 1;           // copies after the first k half

    v16i acc[4][JB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j) acc[i][j] = v16i{};

    // stages 0 .. NS - 1 into the ring, one stage per fenced group
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        put(s);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    wait_vmcnt<(NS - 1) * kOps>();                       // own copies of stage 0
    stage_barrier();
    TlFrags<WB> fr[2];
    tl_issue<WB>(fr[0], ra0, ra1, rb0, rb1);

    // Iteration g: wait for stage g's operands (read in iteration g - 1) and
    // this wave's copies of stage g + 1; barrier (stage g + 1 published, stage
    // g read by all); copy stage g + NS into the slot of stage g; issue the
    // reads of stage g + 1; the MFMAs of stage g.  A tail step is the last
    // stage (g = nkb - 1) and reads and copies nothing.
    auto step = [&](int g, TlFrags<WB>& cur, TlFrags<WB>& nxt, bool tail) {
        tl_wait<WB>(cur);
        const bool more = !tail && g + 1 < nkb;
        if (more) {
            wait_vmcnt<(NS - 2) * kOps>();               // own copies of stage g + 1
            stage_barrier();                             // stage g + 1 published; stage g read by all
            if (!late_copy) put(g + NS);                 // into the slot of stage g
            __atomic_signal_fence(__ATOMIC_SEQ_CST);     // this stage's copies stay in it
            const uint32_t so = (uint32_t)(((g + 1) % NS) * kStage);
            tl_issue<WB>(nxt, ra0 + so, ra1 + so, rb0 + so, rb1 + so);
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            if (kh == 1 && more && late_copy) put(g + NS);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < JB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[2 * i + kh], cur.b[2 * j + kh],
                                                                     acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    int g = 0;
    for (; g + 1 < nkb; g += 2) {                        // the same registers every pass
        step(g, fr[0], fr[1], false);
        step(g + 1, fr[1], fr[0], false);
    }
    if (g < nkb) step(g, fr[0], fr[1], true);
    wait_vmcnt<0>();                                     // no copy outlives the workgroup's LDS

    // Lane l, register 4 q + r of a 32 x 32 block: token l % 32, row
    // 8 q + 4 (l / 32) + r.  Split: this split's int32 partials; unsplit: the
    // epilogue with the tile's scales staged once in LDS.  The tile leaves
    // through the ring in two passes, rows 128 h .. + 127 in pass h: the waves
    // of that row half write their values as [token][128 rows], the 16-byte
    // piece of rows 4 g .. 4 g + 3 of token u at 512 u + 16 (g ^ (u % 32)), then
    // every thread stores whole 512-byte token rows, 32 lanes per token.  (Each
    // lane storing its own 16-byte pieces, 64 tokens per instruction, cost
    // ~20% of the 7B prompt's time.)
    const bool split = P.splits > 1;
    int* const part = split ? P.acc + (int64_t)kidx * P.acc_split : nullptr;
    __shared__ float sws[256], sxs[256];
    if (!split) {
        const int t = (int)threadIdx.x;
        if (t < 256) sws[t] = P.ws[min(n0 + t, P.N - 1)];
        if (t < 64 * WJ) sxs[t] = P.xs[min(t0 + t, P.M - 1)];
    }
    __syncthreads();                                     // every wave is done with the ring
    const bool vec = split ? ((P.acc_ld & 3) == 0 && (P.acc_split & 3) == 0 && ((uintptr_t)P.acc & 15) == 0)
                           : (((uintptr_t)P.Y & 15) == 0 && (P.ldy & 3) == 0 &&
                              (!P.Y2 || (((uintptr_t)P.Y2 & 15) == 0 && (P.ldy2 & 3) == 0)));
    constexpr int kPieces = 64 * WJ * 32;                // 16-byte pieces per pass
    static_assert(64 * WJ * 512 <= NS * kStage, "a pass fits in the ring");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (wn == h) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < JB; ++j) {
                        const int g4 = 8 * i + 2 * q + (lane >> 5);          // rows 4 g4 .. + 3 of the half
                        const int tl = wm * 32 * JB + 32 * j + lrow;         // token in the tile
                        v4i val = v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                        if (!split) {
                            const float4 w4 = *reinterpret_cast<const float4*>(sws + 128 * h + 4 * g4);
                            const float xs = sxs[tl];
                            val = v4i{__float_as_int(epilogue(val[0], w4.x, xs)), __float_as_int(epilogue(val[1], w4.y, xs)),
                                      __float_as_int(epilogue(val[2], w4.z, xs)), __float_as_int(epilogue(val[3], w4.w, xs))};
                        }
                        *reinterpret_cast<v4i*>(ring + tl * 512 + 16 * (g4 ^ (tl & 31))) = val;
                    }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kPieces / (64 * NW); ++u) {
            const int idx = (int)threadIdx.x + 64 * NW * u;
            const int tl = idx >> 5, g4 = idx & 31;
            const int t = t0 + tl, n = n0 + 128 * h + 4 * g4;
            if (t >= P.M || n >= P.N) continue;
            const v4i val = *reinterpret_cast<const v4i*>(ring + tl * 512 + 16 * (g4 ^ (tl & 31)));
            if (split) {
                int* p = part + (int64_t)t * P.acc_ld + n;
                if (vec && n + 3 < P.N) {
                    *reinterpret_cast<v4i*>(p) = val;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < P.N) p[r] = val[r];
                }
                continue;
            }
            float* y = P.Y + (int64_t)t * P.ldy + n;
            float* y2 = P.Y2 ? P.Y2 + (int64_t)t * P.ldy2 + n : nullptr;
            if (vec && n + 3 < P.N) {
                *reinterpret_cast<v4i*>(y) = val;
                if (y2) *reinterpret_cast<v4i*>(y2) = val;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < P.N) {
                        y[r] = __int_as_float(val[r]);
                        if (y2) y2[r] = __int_as_float(val[r]);
                    }
            }
        }
        if (h == 0) __syncthreads();                     // pass 1 overwrites the ring
    }
}

// Workgroup b -> tile (b % 8) * per_xcd + b / 8: the workgroups of one XCD take
// a contiguous range of tiles.  The grid is 8 per_xcd; indices past the last
// tile return at once.
__device__ __forceinline__ int xcd_tile(int per_xcd)
{
    return ((int)blockIdx.x & 7) * per_xcd + ((int)blockIdx.x >> 3);
}

// Waves per tiled workgroup (see tiled_block).
constexpr int kTiledWaves = 8;

// A work unit is (tile, K split), splits fastest.
template <int WJ>
__global__ __launch_bounds__(64 * kTiledWaves) __attribute__((amdgpu_waves_per_eu(kTiledWaves / 4, kTiledWaves / 4)))
void k_gemm_tiled(GemmSet set, int per_xcd)
{
    const int j = xcd_tile(per_xcd);
    if (j >= set.total_tiles) return;
    const GemmProb P = find_prob(set, j);
    const int u = j - P.tile_begin;
    tiled_block<WJ, kTiledWaves>(P, u / P.splits, u % P.splits);
}

// Stack step: with S.partials the K range is split S.splits ways and each unit
// writes its int32 partial tile to the pair's partial buffer.
template <int WJ>
__global__ __launch_bounds__(64 * kTiledWaves) __attribute__((amdgpu_waves_per_eu(kTiledWaves / 4, kTiledWaves / 4)))
void k_gemm_tiled_step(StackStep S, int per_xcd)
{
    const int j = xcd_tile(per_xcd);
    if (j >= S.npairs * S.tile_off[S.nproj] * S.splits) return;
    int local;
    GemmProb P = step_prob(S, j / S.splits, local);
    P.splits = S.splits;
    P.kb_per_split = S.kb_per_split;
    if (S.partials) {
        P.acc = S.pair[(j / S.splits) / S.tile_off[S.nproj]].part;
        P.acc_ld = S.ldp;
        P.acc_split = S.part_stride;
    }
    tiled_block<WJ, kTiledWaves>(P, local, j % S.splits);
}

int tiled_tokens(int64_t M) { return M > 128 ? 256 : 128; }

hipError_t launch_gemm_tiled(const GemmSet& set, int tile_tokens, hipStream_t s)
{
    if (set.total_tiles <= 0) return hipSuccess;
    if (tile_tokens != 256 && tile_tokens != 128) return hipErrorInvalidValue;
    const int per_xcd = (set.total_tiles + 7) / 8;
    const dim3 g(8 * per_xcd), b(64 * kTiledWaves);
    if (tile_tokens == 256) PF_LAUNCH((k_gemm_tiled<4>), g, b, 0, s, set, per_xcd);
    else PF_LAUNCH((k_gemm_tiled<2>), g, b, 0, s, set, per_xcd);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_reduce(set, s);
}

hipError_t launch_gemm_tiled_step(const StackStep& S, int64_t M, hipStream_t s)
{
    if (S.splits < 1 || (S.splits > 1 && !S.partials)) return hipErrorInvalidValue;
    const int tiles = S.npairs * S.tile_off[S.nproj] * S.splits;
    if (tiles <= 0) return hipSuccess;
    const int per_xcd = (tiles + 7) / 8;
    const dim3 g(8 * per_xcd), b(64 * kTiledWaves);
    if (tiled_tokens(M) == 256) PF_LAUNCH((k_gemm_tiled_step<4>), g, b, 0, s, S, per_xcd);
    else PF_LAUNCH((k_gemm_tiled_step<2>), g, b, 0, s, S, per_xcd);
    return hipGetLastError();
}

}  // namespace pf
