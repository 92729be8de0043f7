// Token-by-token KDA prefill with the state held in registers.
//
// The same per-token update as the decode step (see kda_decode.hip), but the
// 128 x 128 fp32 state of a head never leaves the register file between
// tokens: it is loaded once (or zeroed), carried through every token of the
// sequence, and stored once at the end.  This is the plain sequential form of
// the recurrence; the chunked kernel computes the same result blockwise.
//
// Mapping: one workgroup of 256 threads per (sequence, head), lanes laid out as
// in the decode kernel (wave w: columns [32w, 32w+32); lane: 4 columns x 16
// rows).  Packed sequences read their bounds from cu_seqlens on the device.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

template <typename InT, bool RAW>
__global__ __launch_bounds__(256) void prefill_recurrent_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const InT* __restrict__ beta, const float* __restrict__ log_alpha,
    const int32_t* __restrict__ cu_seqlens, int64_t T, int H,
    const StateRefs st, float* __restrict__ o)  // the final state may alias the initial one
{
    const int64_t unit = blockIdx.x;  // n * H + h
    const int64_t n = unit / H;
    const int h = static_cast<int>(unit - n * H);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int rg = lane >> 3;
    const int col = wave * 32 + (lane & 7) * 4;

    int64_t row0, len;
    if (cu_seqlens) {
        row0 = cu_seqlens[n];
        len = static_cast<int64_t>(cu_seqlens[n + 1]) - row0;
    } else {
        row0 = n * T;
        len = T;
    }

    float4 s[16];
    if (const float* S0 = init_state_of(st, n, h, H)) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
            s[m] = *reinterpret_cast<const float4*>(S0 + (rg + 8 * m) * kDim + col);
    } else {
#pragma unroll
        for (int m = 0; m < 16; ++m) s[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    for (int64_t t = 0; t < len; ++t) {
        const int64_t rh = (row0 + t) * H + h;  // (token row, head)
        const int64_t vec = rh * kDim;
        float a[16], kk[16], qq[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int i = rg + 8 * m;
            a[m] = RAW ? alpha_from_logit(log_alpha[vec + i]) : exp_gate(log_alpha[vec + i]);
            kk[m] = widen(k[vec + i]);
            qq[m] = widen(q[vec + i]);
        }
        float bt = widen(beta[rh]);
        if (RAW) {
            // unit q and k: the lane's 16 rows, summed over the 8 row groups
            float ssk = 0.f, ssq = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                ssk += kk[m] * kk[m];
                ssq += qq[m] * qq[m];
            }
            const float ik = inv_norm(xor_sum_rows(ssk)), iq = inv_norm(xor_sum_rows(ssq));
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                kk[m] = unit_round(kk[m] * ik, InT{});
                qq[m] = unit_round(qq[m] * iq, InT{});
            }
            bt = sigmoid_gate(bt);
        }
        const float4 vv = load4(v + vec + col);

        float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
        float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
        float kq = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            s[m].x *= a[m]; s[m].y *= a[m]; s[m].z *= a[m]; s[m].w *= a[m];
            p0 += kk[m] * s[m].x; p1 += kk[m] * s[m].y; p2 += kk[m] * s[m].z; p3 += kk[m] * s[m].w;
            r0 += qq[m] * s[m].x; r1 += qq[m] * s[m].y; r2 += qq[m] * s[m].z; r3 += qq[m] * s[m].w;
            kq += kk[m] * qq[m];
        }
        p0 = xor_sum_rows(p0); p1 = xor_sum_rows(p1); p2 = xor_sum_rows(p2); p3 = xor_sum_rows(p3);
        r0 = xor_sum_rows(r0); r1 = xor_sum_rows(r1); r2 = xor_sum_rows(r2); r3 = xor_sum_rows(r3);
        kq = xor_sum_rows(kq);

        const float u0 = bt * (vv.x - p0), u1 = bt * (vv.y - p1);
        const float u2 = bt * (vv.z - p2), u3 = bt * (vv.w - p3);
        if (rg == 0) {
            *reinterpret_cast<float4*>(o + vec + col) =
                make_float4(r0 + kq * u0, r1 + kq * u1, r2 + kq * u2, r3 + kq * u3);
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            s[m].x += kk[m] * u0; s[m].y += kk[m] * u1; s[m].z += kk[m] * u2; s[m].w += kk[m] * u3;
        }
    }

    if (float* S1 = final_state_of(st, n, h, H)) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
            *reinterpret_cast<float4*>(S1 + (rg + 8 * m) * kDim + col) = s[m];
    }
}

}  // namespace

hipError_t launch_prefill_recurrent(const void* q, const void* k, const void* v,
                                    const void* beta, const float* log_alpha,
                                    const int32_t* cu_seqlens, int64_t n_seq, int64_t T,
                                    int64_t H, const StateRefs& st, float* o, bool bf16,
                                    bool raw, hipStream_t stream)
{
    const int64_t units = n_seq * H;
    if (units <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(units)), block(256);
    const int h = static_cast<int>(H);
    auto go = [&](auto kernel, auto tag) {
        using E = decltype(tag);
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, static_cast<const E*>(q),
                           static_cast<const E*>(k), static_cast<const E*>(v),
                           static_cast<const E*>(beta), log_alpha, cu_seqlens, T, h, st, o);
    };
    if (bf16) {
        if (raw) go(prefill_recurrent_kernel<bf16_t, true>, bf16_t{});
        else go(prefill_recurrent_kernel<bf16_t, false>, bf16_t{});
    } else {
        if (raw) go(prefill_recurrent_kernel<float, true>, 0.f);
        else go(prefill_recurrent_kernel<float, false>, 0.f);
    }
    return hipGetLastError();
}

}  // namespace kda
