// Device-side helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.hpp"

namespace kda {

// bfloat16 as raw storage bits; widening to fp32 is exact.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(bf16_t x) { return __uint_as_float(uint32_t(x.bits) << 16); }

// Four consecutive elements starting at p (p 8-byte aligned for bf16,
// 16-byte aligned for fp32).
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const bf16_t* p)
{
    const uint2 r = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
}

// e^x as 2^(x log2 e) on the hardware exp2 (v_exp_f32).  For the gate values
// used here (x <= 0, |x| up to a few hundred) the relative error is about
// |x| * 2^-24, far below the fp32 state's own rounding over a sequence.
__device__ __forceinline__ float exp_gate(float x)
{
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// The entering / leaving state of head h of sequence n (see StateRefs), or
// NULL for "zeros" / "not written".
__device__ __forceinline__ const float* init_state_of(const StateRefs& r, int64_t n, int h, int64_t H)
{
    if (!r.init) return nullptr;
    int64_t e = n;
    if (r.init_slots) {
        e = r.init_slots[n];
        if (e < 0 || e >= r.n_pool) return nullptr;
    }
    return r.init + (e * H + h) * (kDim * kDim);
}
__device__ __forceinline__ float* final_state_of(const StateRefs& r, int64_t n, int h, int64_t H)
{
    if (!r.fin) return nullptr;
    int64_t e = n;
    if (r.fin_slots) {
        e = r.fin_slots[n];
        if (e < 0 || e >= r.n_pool) return nullptr;
    }
    return r.fin + (e * H + h) * (kDim * kDim);
}

__device__ __forceinline__ float xor_sum_rows(float x)
{
    // sum over lanes that differ in bits 3..5 (the 8 row groups of a wave)
    x += __shfl_xor(x, 8);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

}  // namespace kda
