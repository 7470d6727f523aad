// tiled.hip — the int8 product for chunks of more than 64 tokens (gfx950).
//
// "Batched Prefill" (cellm), §The arithmetic: with hundreds of tokens per chunk
// every weight byte feeds hundreds of multiply-adds, so the product is bound by
// the matrix cores, not by HBM.  The kernel is laid out for v_mfma_i32_32x32x32_i8:
//  * a workgroup of eight waves (two per SIMD) owns 256 weight rows x 64 WJ
//    tokens (WJ = 4 or 2); wave (wn, wm) of the 2 x 4 grid owns 128 rows x
//    16 WJ tokens: 4 x WJ / 2 accumulator blocks of 32 x 32;
//  * a stage is two k-blocks (128 bytes of K) of the tile's weight rows and
//    tokens in LDS as 1 KB fragments of 8 rows x 128 bytes, copied by
//    global_load_lds_dwordx4 with eight consecutive lanes on one row's 128
//    bytes, so every copy instruction reads whole 128-byte lines (whose
//    requests the memory path serves ~30% faster than 64-byte ones); pieces
//    are swizzled so that the MFMA operand reads (one ds_read_b128 each) are
//    conflict-free; the weights sit in a ring of three (256 tokens) or four
//    (128 tokens) stage slots, the tokens in a ring of two, 160 KB in all, one
//    barrier per stage;
//  * each k-block's LDS operand reads for the next k-block are issued between
//    this k-block's MFMAs and waited for inside the same asm block, so no LDS
//    load is ever in flight outside the code that issued it;
//  * workgroups on one XCD (blockIdx % 8) take consecutive tiles, and the token
//    tiles of one band of weight rows are consecutive, so the band is fetched
//    from HBM once into that XCD's L2 and shared.
// Epilogue: y[t][n] = fl(fl(acc) * fl(ws[n] * xs[t])), stored from the
// accumulators as whole 128-byte lines; split products write int32 partials
// instead.
#include "device.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"
#include "problems.hpp"

namespace pf {

// Waves per tiled workgroup.
constexpr int kTiledWaves = 8;

// The epilogue of a tile.  The MFMAs take the tokens as their first operand
// and the weights as their second, so a 32 x 32 accumulator block is indexed
// [token][row]: lane l, register 4 q + r holds token 8 q + 4 (l / 32) + r of
// the block and weight row l % 32.  Output rows are token-major with the
// weight rows contiguous, so each register goes out as one 4-byte store per
// lane that fills two whole 128-byte lines (32 consecutive rows of two
// tokens), straight from the accumulators: no LDS, no barrier.  (Through LDS
// as 256-byte runs, with the weight rows as the first operand, a 256 x 256
// tile took ~10.3 us to leave.)  Split: this split's int32 partials; unsplit:
// y = fl(fl(acc) * fl(ws * xs)).
template <int WJ, int NW>
__device__ __forceinline__ void tiled_store(const GemmProb& P, int n0, int t0, int kidx,
                                            v16i (&acc)[4][2 * WJ / (NW / 2)])
{
    constexpr int JB = 2 * WJ / (NW / 2);
    const bool is_split = P.splits > 1;
    // the lane's place, derived here from the thread index rather than kept
    // live through the main loop
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int col = tid & 31, hi = (tid >> 5) & 1;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = n0 + 128 * (wave >> 2);               // the wave's first weight row
    const int tw = t0 + 32 * JB * (wave & 3);            // the wave's first token
    // the outputs: the split's partials, or the rows and their second copy
    // (without rows to keep, the copy alone; with neither, nothing to store)
    float* y1 = P.Y;
    int64_t ld1 = P.ldy;
    float* y2 = P.Y2;
    if (!is_split && !y1) {
        if (!y2) return;
        y1 = y2;
        ld1 = P.ldy2;
        y2 = nullptr;
    }
    // element e of block (i, j): token tw + 32 j + 8 (e / 4) + 4 hi + e % 4,
    // row nw + 32 i + col.  A full tile (no output past M or N, no second
    // copy) takes its scales and stores at constant offsets from one address.
    const bool full = tw + 32 * JB <= P.M && nw + 128 <= P.N && (is_split || !y2);
    auto tile = [&](auto full_c, auto split_c) {
        constexpr bool F = decltype(full_c)::value, split = decltype(split_c)::value;
        const float* const wp = P.ws + nw + col;
        const float* const xp = P.xs + tw + 4 * hi;
        float ws[4];
        if constexpr (!split) {
#pragma unroll
            for (int i = 0; i < 4; ++i) ws[i] = F ? wp[32 * i] : P.ws[min(nw + 32 * i + col, P.N - 1)];
        }
        int* const out = split ? P.acc + (int64_t)kidx * P.acc_split : reinterpret_cast<int*>(y1);
        const int64_t ld = split ? P.acc_ld : ld1;
        int* const ow = out + (int64_t)(tw + 4 * hi) * ld + nw + col;
        // every scale is loaded before the first store: the memory counter
        // also counts stores, so a later load's wait would wait for them
        float xs[JB][16];
        if constexpr (!split) {
#pragma unroll
            for (int j = 0; j < JB; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int dt = 32 * j + 8 * (e >> 2) + (e & 3);
                    xs[j][e] = F ? xp[dt] : P.xs[min(tw + 4 * hi + dt, P.M - 1)];
                }
        }
#pragma unroll
        for (int j = 0; j < JB; ++j) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int dt = 32 * j + 8 * (e >> 2) + (e & 3);
                const int t = tw + 4 * hi + dt;
                int* const o = ow + (int64_t)dt * ld;
                int v[4];
                if constexpr (split) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = acc[i][j][e];
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = __float_as_int(epilogue(acc[i][j][e], ws[i], xs[j][e]));
                }
                if constexpr (F) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[32 * i] = v[i];
                } else {
                    if (t >= P.M) continue;
                    int* const o2 = (!split && y2) ? reinterpret_cast<int*>(y2) + (int64_t)t * P.ldy2 + nw + col : nullptr;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (nw + 32 * i + col >= P.N) continue;
                        o[32 * i] = v[i];
                        if (o2) o2[32 * i] = v[i];
                    }
                }
            }
        }
    };
    if (is_split) {
        if (full) tile(std::true_type{}, std::true_type{});
        else tile(std::false_type{}, std::true_type{});
    } else {
        if (full) tile(std::true_type{}, std::false_type{});
        else tile(std::false_type{}, std::false_type{});
    }
}

// ---------------------------------------------------------------------------
// Stages of two k-blocks.  A stage is 128 bytes of K of the tile's 256 weight
// rows and 64 WJ tokens in LDS as 1 KB fragments of 8 rows x 128 bytes, so
// every copy instruction reads whole 128-byte lines: eight consecutive lanes
// take one row's 128 bytes (lane l: row l / 8 of the fragment, landing at
// 16 l), with piece c of row r (r counted in the stage) at
// 128 r + 16 (c ^ s(r)), s(r) = (r % 8) ^ ((r / 8) % 2), so that any 16
// consecutive lanes of an operand read touch 16 different 16-byte bank groups
// of a 256-byte span.  A ring of NS stages (two of 64 KB at 256 tokens, three
// of 48 KB at 128), copied NS - 1 stages ahead, one barrier per stage.
//
// Each k-block of a stage is one asm block that issues the LDS reads of the
// next k-block's operands, runs this k-block's MFMAs from registers and waits
// for the reads before it ends, so no load is in flight outside the block
// that issued it.

// One k-block's MFMA operands of a wave: a[2 i + kh] for row block i (32 rows)
// and k half kh (32 bytes), b[2 j + kh] for token block j.
template <int JB>
struct KbOps {
    v4i a[8];
    v4i b[2 * JB];
};

#define PF_RD(dst, adr, off) "ds_read_b128 %[" #dst "], %[" #adr "] offset:" #off "\n"
// the tokens (b) are the first operand, so the result block is [token][row]
#define PF_MF(c, a, b) "v_mfma_i32_32x32x32_i8 %[" #c "], %[" #b "], %[" #a "], %[" #c "]\n"

// kb_half<JB, KH>: n's k half KH <- the operands at ra (row block i at
// + 4096 i) and rb (token block j at + 4096 j), acc += the products of c's k
// half KH, then wait for the reads.  A k-block is two of these, so that c's
// half 0 is dead before n's half 1 is read into its registers.  The compiler
// cannot see the MFMAs inside, so each block first gives the two wait states
// an MFMA needs after a vector ALU write of its sources (the accumulators are
// cleared that way): one s_nop, one read.
template <int JB, int KH>
__device__ __forceinline__ void kb_half(KbOps<JB>& n, const KbOps<JB>& c, v16i (&acc)[4][JB],
                                        uint32_t ra, uint32_t rb)
{
    if constexpr (JB == 2) {
        asm volatile(
            "s_nop 0\n"
            PF_RD(na0, ra, 0) PF_MF(c00, a0, b0)
            PF_RD(nb0, rb, 0) PF_MF(c01, a0, b1)
            PF_RD(na1, ra, 4096) PF_MF(c10, a1, b0)
            PF_RD(nb1, rb, 4096) PF_MF(c11, a1, b1)
            PF_RD(na2, ra, 8192) PF_MF(c20, a2, b0)
            PF_RD(na3, ra, 12288) PF_MF(c21, a2, b1)
            PF_MF(c30, a3, b0)
            PF_MF(c31, a3, b1)
            "s_waitcnt lgkmcnt(0)"
            : [na0] "=&v"(n.a[KH]), [na1] "=&v"(n.a[2 + KH]), [na2] "=&v"(n.a[4 + KH]), [na3] "=&v"(n.a[6 + KH]),
              [nb0] "=&v"(n.b[KH]), [nb1] "=&v"(n.b[2 + KH]),
              [c00] "+v"(acc[0][0]), [c01] "+v"(acc[0][1]), [c10] "+v"(acc[1][0]), [c11] "+v"(acc[1][1]),
              [c20] "+v"(acc[2][0]), [c21] "+v"(acc[2][1]), [c30] "+v"(acc[3][0]), [c31] "+v"(acc[3][1])
            : [a0] "v"(c.a[KH]), [a1] "v"(c.a[2 + KH]), [a2] "v"(c.a[4 + KH]), [a3] "v"(c.a[6 + KH]),
              [b0] "v"(c.b[KH]), [b1] "v"(c.b[2 + KH]), [ra] "v"(ra), [rb] "v"(rb));
    } else {
        asm volatile(
            "s_nop 0\n"
            PF_RD(na0, ra, 0) PF_MF(c0, a0, b0)
            PF_RD(nb0, rb, 0) PF_MF(c1, a1, b0)
            PF_RD(na1, ra, 4096) PF_MF(c2, a2, b0)
            PF_RD(na2, ra, 8192) PF_MF(c3, a3, b0)
            PF_RD(na3, ra, 12288)
            "s_waitcnt lgkmcnt(0)"
            : [na0] "=&v"(n.a[KH]), [na1] "=&v"(n.a[2 + KH]), [na2] "=&v"(n.a[4 + KH]), [na3] "=&v"(n.a[6 + KH]),
              [nb0] "=&v"(n.b[KH]),
              [c0] "+v"(acc[0][0]), [c1] "+v"(acc[1][0]), [c2] "+v"(acc[2][0]), [c3] "+v"(acc[3][0])
            : [a0] "v"(c.a[KH]), [a1] "v"(c.a[2 + KH]), [a2] "v"(c.a[4 + KH]), [a3] "v"(c.a[6 + KH]),
              [b0] "v"(c.b[KH]), [ra] "v"(ra), [rb] "v"(rb));
    }
}

// kb_step: n <- the next k-block's operands (k half kh at ra_kh, rb_kh),
// acc += the products of c.
template <int JB>
__device__ __forceinline__ void kb_step(KbOps<JB>& n, const KbOps<JB>& c, v16i (&acc)[4][JB],
                                        uint32_t ra0, uint32_t ra1, uint32_t rb0, uint32_t rb1)
{
    kb_half<JB, 0>(n, c, acc, ra0, rb0);
    kb_half<JB, 1>(n, c, acc, ra1, rb1);
}

// kb_read: n <- the operands at (ra0, ra1, rb0, rb1), waited for.
template <int JB>
__device__ __forceinline__ void kb_read(KbOps<JB>& n, uint32_t ra0, uint32_t ra1, uint32_t rb0, uint32_t rb1)
{
    if constexpr (JB == 2) {
        asm volatile(
            PF_RD(na0, ra0, 0) PF_RD(na1, ra1, 0) PF_RD(na2, ra0, 4096) PF_RD(na3, ra1, 4096)
            PF_RD(na4, ra0, 8192) PF_RD(na5, ra1, 8192) PF_RD(na6, ra0, 12288) PF_RD(na7, ra1, 12288)
            PF_RD(nb0, rb0, 0) PF_RD(nb1, rb1, 0) PF_RD(nb2, rb0, 4096) PF_RD(nb3, rb1, 4096)
            "s_waitcnt lgkmcnt(0)"
            : [na0] "=&v"(n.a[0]), [na1] "=&v"(n.a[1]), [na2] "=&v"(n.a[2]), [na3] "=&v"(n.a[3]),
              [na4] "=&v"(n.a[4]), [na5] "=&v"(n.a[5]), [na6] "=&v"(n.a[6]), [na7] "=&v"(n.a[7]),
              [nb0] "=&v"(n.b[0]), [nb1] "=&v"(n.b[1]), [nb2] "=&v"(n.b[2]), [nb3] "=&v"(n.b[3])
            : [ra0] "v"(ra0), [ra1] "v"(ra1), [rb0] "v"(rb0), [rb1] "v"(rb1));
    } else {
        asm volatile(
            PF_RD(na0, ra0, 0) PF_RD(na1, ra1, 0) PF_RD(na2, ra0, 4096) PF_RD(na3, ra1, 4096)
            PF_RD(na4, ra0, 8192) PF_RD(na5, ra1, 8192) PF_RD(na6, ra0, 12288) PF_RD(na7, ra1, 12288)
            PF_RD(nb0, rb0, 0) PF_RD(nb1, rb1, 0)
            "s_waitcnt lgkmcnt(0)"
            : [na0] "=&v"(n.a[0]), [na1] "=&v"(n.a[1]), [na2] "=&v"(n.a[2]), [na3] "=&v"(n.a[3]),
              [na4] "=&v"(n.a[4]), [na5] "=&v"(n.a[5]), [na6] "=&v"(n.a[6]), [na7] "=&v"(n.a[7]),
              [nb0] "=&v"(n.b[0]), [nb1] "=&v"(n.b[1])
            : [ra0] "v"(ra0), [ra1] "v"(ra1), [rb0] "v"(rb0), [rb1] "v"(rb1));
    }
}


// kb_last: acc += the products of c (the last k-block: nothing to read).  It
// ends with 20 wait states, more than a 16-pass MFMA needs before a vector
// ALU instruction may read its result, since the compiler does not see these
// MFMAs when it places the epilogue's reads of acc.
template <int JB>
__device__ __forceinline__ void kb_last(const KbOps<JB>& c, v16i (&acc)[4][JB])
{
    if constexpr (JB == 2) {
        asm volatile(
            "s_nop 1\n"
            PF_MF(c00, a0, b0) PF_MF(c01, a0, b2) PF_MF(c10, a2, b0) PF_MF(c11, a2, b2)
            PF_MF(c20, a4, b0) PF_MF(c21, a4, b2) PF_MF(c30, a6, b0) PF_MF(c31, a6, b2)
            PF_MF(c00, a1, b1) PF_MF(c01, a1, b3) PF_MF(c10, a3, b1) PF_MF(c11, a3, b3)
            PF_MF(c20, a5, b1) PF_MF(c21, a5, b3) PF_MF(c30, a7, b1) PF_MF(c31, a7, b3)
            "s_nop 7\n s_nop 7\n s_nop 3"
            : [c00] "+v"(acc[0][0]), [c01] "+v"(acc[0][1]), [c10] "+v"(acc[1][0]), [c11] "+v"(acc[1][1]),
              [c20] "+v"(acc[2][0]), [c21] "+v"(acc[2][1]), [c30] "+v"(acc[3][0]), [c31] "+v"(acc[3][1])
            : [a0] "v"(c.a[0]), [a1] "v"(c.a[1]), [a2] "v"(c.a[2]), [a3] "v"(c.a[3]),
              [a4] "v"(c.a[4]), [a5] "v"(c.a[5]), [a6] "v"(c.a[6]), [a7] "v"(c.a[7]),
              [b0] "v"(c.b[0]), [b1] "v"(c.b[1]), [b2] "v"(c.b[2]), [b3] "v"(c.b[3]));
    } else {
        asm volatile(
            "s_nop 1\n"
            PF_MF(c0, a0, b0) PF_MF(c1, a2, b0) PF_MF(c2, a4, b0) PF_MF(c3, a6, b0)
            PF_MF(c0, a1, b1) PF_MF(c1, a3, b1) PF_MF(c2, a5, b1) PF_MF(c3, a7, b1)
            "s_nop 7\n s_nop 7\n s_nop 3"
            : [c0] "+v"(acc[0][0]), [c1] "+v"(acc[1][0]), [c2] "+v"(acc[2][0]), [c3] "+v"(acc[3][0])
            : [a0] "v"(c.a[0]), [a1] "v"(c.a[1]), [a2] "v"(c.a[2]), [a3] "v"(c.a[3]),
              [a4] "v"(c.a[4]), [a5] "v"(c.a[5]), [a6] "v"(c.a[6]), [a7] "v"(c.a[7]),
              [b0] "v"(c.b[0]), [b1] "v"(c.b[1]));
    }
}

#undef PF_RD
#undef PF_MF

// One 256 x 64 WJ output tile of problem P (tile `local`, token tiles fastest)
// by eight waves in a 2 x 4 grid: wave (wn, wm) owns rows 128 wn .. + 127 and
// tokens 32 JB wm .. + 32 JB - 1 (JB = WJ / 2 blocks of 32): 4 x JB
// accumulator blocks of 32 x 32.  Stage s is k-blocks 2 s, 2 s + 1 of this
// split, held in two rings: the weights in NSW slots of 32 KB (fragments
// 0 .. 31), copied NSW - 1 stages ahead, the tokens in NST slots of 8 WJ KB
// (fragments 0 .. 8 WJ - 1), copied NST - 1 ahead, 160 KB in all; wave w
// copies fragments w + 8 h of each.  The weights come from HBM or the
// Infinity Cache, the tokens mostly from L2, so the weights get the longer
// lead (three weight slots against two: the 7B prompt 16.7 -> 16.2 ms,
// 38400 x 4096 x 512 143 -> 134 us).  Iteration g:
//   k-block 2 g: read k-block 2 g + 1 of stage g, MFMAs of 2 g;
//   wait for this wave's copies of stage g + 1; barrier (stage g + 1
//   published, stage g read by all); copy the tokens of stage g + NST, then
//   the weights of stage g + NSW, into stage g's slots;
//   k-block 2 g + 1: read k-block 2 g + 2 of stage g + 1, MFMAs of 2 g + 1.
// Tokens before weights: waiting for the tokens of stage g + 1 leaves only
// the newest weights in flight, and the weights of stage g + 1, copied
// earlier, have landed too.  Every iteration issues the same copies (k-blocks
// past the end are clamped to the last one and land in free slots, never
// read), so every wait is a constant.
template <int WJ>
__device__ __forceinline__ void tiled_block(const GemmProb& P, int local, int kidx)
{
    constexpr int NW = kTiledWaves;
    constexpr int NSW = WJ == 4 ? 3 : 4, NST = 2;
    constexpr int JB = WJ / 2;
    constexpr int kFa = 32, kFb = 8 * WJ;                // fragments per stage
    constexpr int kWst = kFa * 1024, kTst = kFb * 1024;
    constexpr int ka = kFa / NW, kb = kFb / NW;          // copies per wave per stage
    constexpr int kRing = NSW * kWst + NST * kTst;
    static_assert(kRing <= 160 * 1024, "LDS");
    static_assert(ka + (NST - 1) * (ka + kb) <= 63, "vmcnt range");
        __shared__ __attribute__((aligned(16))) int8_t ring[kRing];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tm = local % P.tiles_m, tn = local / P.tiles_m;
    const int n0 = tn * 256, t0 = tm * 64 * WJ;
    const int kb0 = kidx * P.kb_per_split;
    const int nkb = min(P.kb_per_split, (P.K >> 6) - kb0);
    const int nst = (nkb + 1) >> 1;
    const int crow = lane >> 3;
    const int pc = (lane & 7) ^ crow ^ (wave & 1);
    const int phalf = pc >> 2;
    const int pof = (pc & 3) << 4;
    // 32-bit offsets from the matrices' bases (weights and tokens are each
    // under 2 GiB), so a copy's address is one register plus a uniform base
    uint32_t aoff[ka], boff[kb];
#pragma unroll
    for (int h = 0; h < ka; ++h)
        aoff[h] = (uint32_t)min(n0 + 8 * (wave + NW * h) + crow, P.N - 1) * (uint32_t)P.K + (uint32_t)(kb0 * 64 + pof);
#pragma unroll
    for (int h = 0; h < kb; ++h)
        boff[h] = (uint32_t)min(t0 + 8 * (wave + NW * h) + crow, P.M - 1) * (uint32_t)P.ldx + (uint32_t)(kb0 * 64 + pof);
    const uint32_t ring0 = lds_addr(ring);
    int8_t* const tring = ring + NSW * kWst;

    auto put_w = [&](int s) {
        int8_t* slot = ring + (s % NSW) * kWst;
        const uint32_t ko = (uint32_t)min(2 * s + phalf, nkb - 1) * 64u;
#pragma unroll
        for (int h = 0; h < ka; ++h) dma16(P.W + (aoff[h] + ko), slot + (wave + NW * h) * 1024);
    };
    auto put_t = [&](int s) {
        int8_t* slot = tring + (s % NST) * kTst;
        const uint32_t ko = (uint32_t)min(2 * s + phalf, nkb - 1) * 64u;
#pragma unroll
        for (int h = 0; h < kb; ++h) dma16(P.X + (boff[h] + ko), slot + (wave + NW * h) * 1024);
    };

    const int r = lane & 31;
    const int sr = (r & 7) ^ ((r >> 3) & 1);
    const uint32_t lo = (uint32_t)(128 * r + 16 * ((lane >> 5) ^ sr));
    const int wn = wave >> 2, wm = wave & 3;
    const uint32_t xa = (uint32_t)(wn * 128 * 128) + lo;
    const uint32_t xb = (uint32_t)(NSW * kWst + wm * JB * 32 * 128) + lo;
    auto ra = [&](int s, int q) { return ring0 + (uint32_t)((s % NSW) * kWst) + (xa ^ (uint32_t)(32 * q)); };
    auto rb = [&](int s, int q) { return ring0 + (uint32_t)((s % NST) * kTst) + (xb ^ (uint32_t)(32 * q)); };

    v16i acc[4][JB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j) acc[i][j] = v16i{};

    // the copies of iterations -NSW .. -1
#pragma unroll
    for (int g = -NSW; g < 0; ++g) {
        if (g + NST >= 0) put_t(g + NST);
        put_w(g + NSW);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    wait_vmcnt<ka + (NST - 1) * (ka + kb)>();            // own copies of stage 0
    stage_barrier();
    KbOps<JB> c0, c1;
    kb_read<JB>(c0, ra(0, 0), ra(0, 1), rb(0, 0), rb(0, 1));

    for (int g = 0; g + 1 < nst; ++g) {
        kb_step<JB>(c1, c0, acc, ra(g, 2), ra(g, 3), rb(g, 2), rb(g, 3));
        wait_vmcnt<ka + (NST - 2) * (ka + kb)>();        // own copies of stage g + 1
        stage_barrier();                                 // stage g + 1 published; stage g read by all
        put_t(g + NST);                                  // into the slots of stage g
        put_w(g + NSW);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        kb_step<JB>(c0, c1, acc, ra(g + 1, 0), ra(g + 1, 1), rb(g + 1, 0), rb(g + 1, 1));
    }
    // the last stage: with an odd k-block count its second k-block's token
    // operands are replaced by zeros, so it adds nothing
    {
        const int g = nst - 1;
        kb_step<JB>(c1, c0, acc, ra(g, 2), ra(g, 3), rb(g, 2), rb(g, 3));
        if (2 * nst != nkb) {
#pragma unroll
            for (int j = 0; j < 2 * JB; ++j) c1.b[j] = v4i{0, 0, 0, 0};
        }
        kb_last<JB>(c1, acc);
    }
    wait_vmcnt<0>();                                     // no copy outlives the workgroup's LDS
    tiled_store<WJ, NW>(P, n0, t0, kidx, acc);
}

// Workgroup b -> tile (b % 8) * per_xcd + b / 8: the workgroups of one XCD take
// a contiguous range of tiles.  The grid is 8 per_xcd; indices past the last
// tile return at once.
__device__ __forceinline__ int xcd_tile(int per_xcd)
{
    return ((int)blockIdx.x & 7) * per_xcd + ((int)blockIdx.x >> 3);
}

// A work unit is (tile, K split), splits fastest.
template <int WJ>
__global__ __launch_bounds__(64 * kTiledWaves) __attribute__((amdgpu_waves_per_eu(kTiledWaves / 4, kTiledWaves / 4)))
void k_gemm_tiled(GemmSet set, int per_xcd)
{
    const int j = xcd_tile(per_xcd);
    if (j >= set.total_tiles) return;
    const GemmProb P = find_prob(set, j);
    const int u = j - P.tile_begin;
    tiled_block<WJ>(P, u / P.splits, u % P.splits);
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
    tiled_block<WJ>(P, local, j % S.splits);
}

int tiled_tokens(int64_t M) { return M > 128 ? 256 : 128; }

hipError_t launch_gemm_tiled(const GemmSet& set, int tile_tokens, hipStream_t s)
{
    if (set.total_tiles <= 0) return hipSuccess;
    if (tile_tokens != 256 && tile_tokens != 128) return hipErrorInvalidValue;
    for (int i = 0; i < set.nprob; ++i)                  // 32-bit copy offsets
        if ((uint64_t)set.p[i].N * (uint64_t)set.p[i].K >= (1ull << 32) ||
            (uint64_t)set.p[i].M * (uint64_t)set.p[i].ldx >= (1ull << 32))
            return hipErrorInvalidValue;
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
    for (int j = 0; j < S.nproj; ++j)                    // 32-bit copy offsets
        if ((uint64_t)S.rows[j] * (uint64_t)S.K >= (1ull << 32)) return hipErrorInvalidValue;
    if ((uint64_t)M * (uint64_t)S.ldx >= (1ull << 32)) return hipErrorInvalidValue;
    const int tiles = S.npairs * S.tile_off[S.nproj] * S.splits;
    if (tiles <= 0) return hipSuccess;
    const int per_xcd = (tiles + 7) / 8;
    const dim3 g(8 * per_xcd), b(64 * kTiledWaves);
    if (tiled_tokens(M) == 256) PF_LAUNCH((k_gemm_tiled_step<4>), g, b, 0, s, S, per_xcd);
    else PF_LAUNCH((k_gemm_tiled_step<2>), g, b, 0, s, S, per_xcd);
    return hipGetLastError();
}

}  // namespace pf
