// device.hpp — device-side building blocks shared by the libprefill kernels.
//
// Everything here is compiled for gfx950 (CDNA4) with -ffp-contract=off and
// without fast-math: each float expression is one IEEE binary32 operation
// rounded to nearest even, in the written order, so the quantiser and the
// epilogue give the same bits as their plain per-token definition.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pf {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// One 128-bit load / store.
__device__ __forceinline__ v4i ld16(const int8_t* p) { return *reinterpret_cast<const v4i*>(p); }
__device__ __forceinline__ void st16(int8_t* p, v4i v) { *reinterpret_cast<v4i*>(p) = v; }
// A 128-bit load marked non-temporal: weights streamed once per use.
__device__ __forceinline__ v4i ld16_nt(const int8_t* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

// Epilogue of one output: fl( fl((float)acc) * fl(w_scale * a_scale) ), the
// scale product taken first.
__device__ __forceinline__ float epilogue(int acc, float w_scale, float a_scale)
{
    const float scale = w_scale * a_scale;
    const float a = (float)acc;
    return a * scale;
}

// One int8 code: clamp(roundf(fl(x / s)), -127, 127); roundf rounds halves away
// from zero.  s != 0.
__device__ __forceinline__ int quant_code(float x, float s)
{
    float r = roundf(x / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

}  // namespace pf
