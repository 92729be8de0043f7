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

// The same four elements as raw storage (for a load issued ahead of its
// use), and their widening.
__device__ __forceinline__ float4 load4_raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ uint2 load4_raw(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ float4 widen4(float4 r) { return r; }
__device__ __forceinline__ float4 widen4(uint2 r)
{
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
}
// Two consecutive elements as raw storage (p 4-byte aligned for bf16, 8-byte
// aligned for fp32), and their widening.
__device__ __forceinline__ float2 load2_raw(const float* p) { return *reinterpret_cast<const float2*>(p); }
__device__ __forceinline__ uint32_t load2_raw(const bf16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ float2 widen2(float2 r) { return r; }
__device__ __forceinline__ float2 widen2(uint32_t r)
{
    return make_float2(__uint_as_float(r << 16), __uint_as_float(r & 0xffff0000u));
}

// e^x as 2^(x log2 e) on the hardware exp2 (v_exp_f32).  For the gate values
// used here (x <= 0, |x| up to a few hundred) the relative error is about
// |x| * 2^-24, far below the fp32 state's own rounding over a sequence.
__device__ __forceinline__ float exp_gate(float x)
{
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Raw-input preparation (see kda.h, the *_raw entry points): q and k become
// unit vectors per (token, head), rounded to bf16 when the inputs are bf16;
// beta = sigmoid(b); log alpha = -softplus(a), i.e. alpha = 1 / (1 + e^a).
__device__ __forceinline__ float unit_round(float x, bf16_t) { return (float)(__bf16)x; }
__device__ __forceinline__ float unit_round(float x, float) { return x; }
__device__ __forceinline__ float inv_norm(float sum_sq) { return sum_sq > 0.f ? rsqrtf(sum_sq) : 0.f; }
__device__ __forceinline__ float sigmoid_gate(float b) { return 1.f / (1.f + __expf(-b)); }
__device__ __forceinline__ float alpha_from_logit(float a) { return 1.f / (1.f + __expf(a)); }
// log2 alpha = -softplus(a) / ln 2 = -log2(1 + 2^t) with t = a log2 e, as
// -(max(t, 0) + log2(1 + y)) with y = 2^-|t| in (0, 1] (no overflow), on the
// hardware exp2 / log2.  log2(1 + y) is taken as log2(u) * y / (u - 1) with
// u = fl(1 + y): the rounding of u cancels between the two factors, so tiny y
// keep their relative accuracy (Goldberg, "What every computer scientist
// should know about floating-point arithmetic", the log(1 + x) theorem);
// u == 1 means y is below half an ulp of 1 and log2(1 + y) = y log2 e.
__device__ __forceinline__ float log2_alpha_from_logit(float a)
{
    const float t = a * 1.4426950408889634f;
    const float y = __builtin_amdgcn_exp2f(-fabsf(t));
    const float u = 1.f + y;
    // both forms, then a select: a conditional expression with the logarithm
    // in one arm is compiled as a branch around it
    const float tiny = y * 1.4426950408889634f;
    const float rest = __builtin_amdgcn_logf(u) * (y * __builtin_amdgcn_rcpf(u - 1.f));
    const float l = u == 1.f ? tiny : rest;
    return -(fmaxf(t, 0.f) + l);
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

// Sum over the 8 lanes that differ in lane bits 3..5 (the 8 row groups of a
// wave), without the LDS crossbar: lane l ^ 8 through a DPP rotate by 8 within
// each 16-lane row; l ^ 16 and l ^ 32 through the gfx950 lane-swap
// instructions.  permlane16_swap(x, x) returns, in every lane, the values of
// the even and of the odd row of its row pair (their sum is x[l] + x[l ^ 16]);
// permlane32_swap(x, x) those of the lower and upper half-wave.
__device__ __forceinline__ float xor_sum_rows(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

// Lane mapping shared by the token-by-token kernels (decode, draft tokens,
// token-recurrent prefill): one 256-thread workgroup per head; wave w owns
// state columns 32w .. 32w+31 and lane l the 16 consecutive rows
// 16*(l >> 3) .. +15 of columns 32w + 4*(l & 7) .. +3, 64 values in registers.
//
// One token of the recurrence on a lane's share of the state: S' = Diag(a) S;
// p = S'^T k summed over all 128 rows (the other row groups through
// xor_sum_rows); u = beta (v - p); S <- S' + k u^T; then o = S^T q from the
// updated state.  a, k and q point at the lane's 16 rows of the token's gate,
// key and query staged in LDS (16-byte aligned); they are read where used
// rather than held in registers, which keeps the kernels at four waves per
// SIMD.  vt holds the lane's 4 columns of v.  With RAW, k and q are raw
// projections: each is scaled to a unit vector (rounded to bf16 for bf16
// inputs) as it is read.  Returns the lane's 4 columns of o.
template <typename InT, bool RAW>
__device__ __forceinline__ float4 token_update(float4 (&s)[16], const float* a, const float* k,
                                               const float* q, float bt, float4 vt)
{
    float ik = 1.f, iq = 1.f;
    if (RAW) {
        float ssk = 0.f, ssq = 0.f;
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            const float4 k4 = *reinterpret_cast<const float4*>(k + 4 * m4);
            const float4 q4 = *reinterpret_cast<const float4*>(q + 4 * m4);
            ssk += k4.x * k4.x + k4.y * k4.y + k4.z * k4.z + k4.w * k4.w;
            ssq += q4.x * q4.x + q4.y * q4.y + q4.z * q4.z + q4.w * q4.w;
        }
        ik = inv_norm(xor_sum_rows(ssk));
        iq = inv_norm(xor_sum_rows(ssq));
    }
    auto key = [&](float x) { return RAW ? unit_round(x * ik, InT{}) : x; };
    auto query = [&](float x) { return RAW ? unit_round(x * iq, InT{}) : x; };
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
        const float4 a4 = *reinterpret_cast<const float4*>(a + 4 * m4);
        const float4 k4 = *reinterpret_cast<const float4*>(k + 4 * m4);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
        const float kv[4] = {key(k4.x), key(k4.y), key(k4.z), key(k4.w)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * m4 + i;
            s[m].x *= av[i]; s[m].y *= av[i]; s[m].z *= av[i]; s[m].w *= av[i];
            p0 += kv[i] * s[m].x; p1 += kv[i] * s[m].y; p2 += kv[i] * s[m].z; p3 += kv[i] * s[m].w;
        }
    }
    p0 = xor_sum_rows(p0); p1 = xor_sum_rows(p1); p2 = xor_sum_rows(p2); p3 = xor_sum_rows(p3);
    const float u0 = bt * (vt.x - p0), u1 = bt * (vt.y - p1);
    const float u2 = bt * (vt.z - p2), u3 = bt * (vt.w - p3);
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
        const float4 k4 = *reinterpret_cast<const float4*>(k + 4 * m4);
        const float4 q4 = *reinterpret_cast<const float4*>(q + 4 * m4);
        const float kv[4] = {key(k4.x), key(k4.y), key(k4.z), key(k4.w)};
        const float qv[4] = {query(q4.x), query(q4.y), query(q4.z), query(q4.w)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * m4 + i;
            s[m].x += kv[i] * u0; s[m].y += kv[i] * u1; s[m].z += kv[i] * u2; s[m].w += kv[i] * u3;
            o0 += qv[i] * s[m].x; o1 += qv[i] * s[m].y; o2 += qv[i] * s[m].z; o3 += qv[i] * s[m].w;
        }
    }
    return make_float4(xor_sum_rows(o0), xor_sum_rows(o1), xor_sum_rows(o2), xor_sum_rows(o3));
}

}  // namespace kda
