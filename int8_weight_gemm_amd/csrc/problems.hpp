// problems.hpp — device-side lookup of the product a workgroup works on.
#pragma once

#include "device.hpp"
#include "kernels.hpp"

namespace pf {

// Problem lookup inside a grouped launch.  Static indices only, so the
// descriptors stay in scalar registers.
__device__ __forceinline__ GemmProb find_prob(const GemmSet& set, int bid)
{
    GemmProb P = set.p[0];
#pragma unroll
    for (int j = 1; j < kMaxProbs; ++j)
        if (j < set.nprob && bid >= set.p[j].tile_begin) P = set.p[j];
    return P;
}

// Problem of a stack step: workgroup bid -> (pair, projection, tile).
__device__ __forceinline__ GemmProb step_prob(const StackStep& S, int bid, int& local)
{
    const int per = S.tile_off[S.nproj];
    const int pi = bid / per;
    const int lp = bid - pi * per;
    int j = 0;
#pragma unroll
    for (int q = 1; q < 6; ++q)
        if (q < S.nproj && lp >= S.tile_off[q]) j = q;
    local = lp - S.tile_off[j];
    const StepPair& pp = S.pair[pi];
    GemmProb P;
    P.W = pp.W[j];
    P.ws = pp.ws[j];
    P.X = pp.X;
    P.xs = pp.xs;
    P.Y = ((S.nostore >> j) & 1u) ? nullptr : pp.Y + S.yoff[j];
    P.Y2 = pp.Y2;
    P.ldy2 = S.ldy2;
    if (float* kv = step_kv(S, pp, j)) {
        P.Y2 = kv;
        P.ldy2 = S.ldkv;
    }
    P.acc = nullptr;
    P.acc_ld = 0;
    P.acc_split = 0;
    P.ldx = S.ldx;
    P.ldy = S.ldy;
    P.N = S.rows[j];
    P.K = S.K;
    P.M = pp.M;
    P.tiles_n = 0;
    P.tiles_m = S.tiles_m;
    P.splits = 1;
    P.kb_per_split = S.K >> 6;
    P.tile_begin = 0;
    return P;
}

__device__ __forceinline__ void store_out(const GemmProb& P, int t, int n, float v)
{
    if (P.Y) P.Y[(int64_t)t * P.ldy + n] = v;
    if (P.Y2) P.Y2[(int64_t)t * P.ldy2 + n] = v;
}

}  // namespace pf
