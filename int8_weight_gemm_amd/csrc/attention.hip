// attention.hip — causal attention over the prompt's K/V cache (gfx950).
//
// "Batched Prefill" (cellm), §What Stays Sequential: only the linear layers are
// batched; attention is sequential over positions and runs per position inside
// each chunk.  "Single-pass prefill", "The fix": position t attends over the
// K/V history of its layer, positions 0 .. t, which every earlier position has
// already written.  The arithmetic is fixed so that the result is bit-exact
// with a per-token evaluation:
//   per head (d values): s_j = fl(dot(q, K_j) * c), the dot summed in ascending
//   index from +0 with each product and sum rounded on its own, c = fl(1/fl(sqrt d));
//   m = max_j s_j; z_j = expf_cr(fl(s_j - m)); S = z_0 + z_1 + ... in ascending j;
//   p_j = fl(z_j / S); out_i = sum over ascending j of fl(p_j * V_j,i) from +0;
// then the attention row is quantised per token (as every layer input is).
//
// One workgroup per token, one wave per head (a wave takes several heads when
// there are more than 16).  Every score is one lane's sequential chain of d
// products; a wave scores 64 positions at a time.  The three passes (maximum,
// normaliser, weighted sum) recompute the scores rather than keep them, so no
// buffer grows with the prompt; the weighted sum turns the wave around, lanes
// over the head's values, each a sequential chain over positions.
#include "device.hpp"
#include "expf_cr.hpp"
#include "kernels.hpp"

namespace pf {

// s_j = fl(dot(q, K_j) * c): q from LDS (every lane reads the same address),
// K_j from the cache, four values per load, summed one by one in order.
__device__ __forceinline__ float attn_score(const float* qs, const float* kr, int d, float c)
{
    float acc = 0.0f;
    for (int i = 0; i < d; i += 4) {
        const float4 k4 = *reinterpret_cast<const float4*>(kr + i);
        const float4 q4 = *reinterpret_cast<const float4*>(qs + i);
        acc = acc + q4.x * k4.x;
        acc = acc + q4.y * k4.y;
        acc = acc + q4.z * k4.z;
        acc = acc + q4.w * k4.w;
    }
    return acc * c;
}

__global__ __launch_bounds__(1024) void k_attention(AttnStep S)
{
    __shared__ __attribute__((aligned(16))) float row[kAttnMaxH];          // the attention row
    __shared__ __attribute__((aligned(16))) float qsh[16][kAttnMaxD];      // q of each wave's head
    __shared__ float xb[16][64];                                          // a block's weights
    __shared__ float red[16];
    const int pi = (int)blockIdx.x / S.max_m, tt = (int)blockIdx.x % S.max_m;
    const AttnPair& P = S.pair[pi];
    if (tt >= P.M) return;                               // the whole workgroup
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int t = P.pos0 + tt;                           // this token's position
    const int d = S.d;
    const float* q = P.q + (int64_t)tt * S.ldq;
    float* qs = qsh[wave];
    float* xw = xb[wave];

    for (int hd = wave; hd < S.n_heads; hd += nw) {
        const int c0 = hd * d;
        for (int i = lane; i < d; i += 64) qs[i] = q[c0 + i];
        __builtin_amdgcn_wave_barrier();
        const float* K = P.K + c0;
        const float* V = P.V + c0;
        // pass 1: the maximum score
        float m = -__builtin_huge_valf();
        for (int jb = 0; jb <= t; jb += 64) {
            const int j = jb + lane;
            if (j <= t) m = fmaxf(m, attn_score(qs, K + (int64_t)j * S.ldkv, d, S.scale));
        }
        m = wave_max(m);
        // pass 2: S, the z_j summed in ascending j (every lane reads each block's
        // z from LDS in order and keeps the same running sum)
        float Ssum = 0.0f;
        for (int jb = 0; jb <= t; jb += 64) {
            const int j = jb + lane;
            const int nb = min(64, t + 1 - jb);
            if (j <= t) xw[lane] = expf_cr(attn_score(qs, K + (int64_t)j * S.ldkv, d, S.scale) - m);
            __builtin_amdgcn_wave_barrier();
            for (int u = 0; u < nb; ++u) Ssum = Ssum + xw[u];
            __builtin_amdgcn_wave_barrier();
        }
        // pass 3: p_j = fl(z_j / S), then out_i = sum over ascending j of
        // fl(p_j * V_j,i) with lanes over i (up to four values of the head each)
        float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int jb = 0; jb <= t; jb += 64) {
            const int j = jb + lane;
            const int nb = min(64, t + 1 - jb);
            if (j <= t) xw[lane] = expf_cr(attn_score(qs, K + (int64_t)j * S.ldkv, d, S.scale) - m) / Ssum;
            __builtin_amdgcn_wave_barrier();
            for (int u = 0; u < nb; ++u) {
                const float p = xw[u];
                const float* vr = V + (int64_t)(jb + u) * S.ldkv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = lane + 64 * r;
                    if (i < d) o[r] = o[r] + p * vr[i];
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (lane + 64 * r < d) row[c0 + lane + 64 * r] = o[r];
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    // quantise the row: amax (exact), s = fl(amax / 127), codes
    float amax = 0.0f;
    for (int i = threadIdx.x; i < S.H; i += blockDim.x) amax = fmaxf(amax, fabsf(row[i]));
    amax = wave_max(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = red[0];
    for (int w = 1; w < nw; ++w) amax = fmaxf(amax, red[w]);
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) P.sao[tt] = s;
    int8_t* qrow = P.ao + (int64_t)tt * S.H;
    for (int i = threadIdx.x; i < S.H; i += blockDim.x)
        qrow[i] = (int8_t)(s != 0.0f ? quant_code(row[i], s) : 0);
}

hipError_t launch_attention(const AttnStep& S, hipStream_t s)
{
    if (S.npairs <= 0 || S.max_m <= 0) return hipSuccess;
    if (S.H > kAttnMaxH || S.d > kAttnMaxD || S.d % 4 != 0 || S.n_heads * S.d != S.H)
        return hipErrorInvalidValue;
    const int nw = S.n_heads < 16 ? S.n_heads : 16;
    PF_LAUNCH(k_attention, dim3(S.npairs * S.max_m), dim3(64 * nw), 0, s, S);
    return hipGetLastError();
}

}  // namespace pf
