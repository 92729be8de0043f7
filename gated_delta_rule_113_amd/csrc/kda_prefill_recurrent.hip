// Token-by-token KDA prefill with the state held in registers.
//
// The same per-token update as the decode step (see kda_decode.hip), but the
// 128 x 128 fp32 state of a head never leaves the register file between
// tokens: it is loaded once (or zeroed), carried through every token of the
// sequence, and stored once at the end.  This is the plain sequential form of
// the recurrence; the chunked kernel computes the same result blockwise.  It
// serves fp32 inputs (not exact in bf16, so not fit for the bf16 matrix
// path) and short sequences, where the chunked kernel's fixed cost per chunk
// dominates.
//
// Mapping: one workgroup of 256 threads per (sequence, head), lanes laid out as
// in the decode kernel.  Inputs are staged through LDS in batches of TB
// tokens: each thread requests one gate and one value element (threads
// 0..127) or one key and one query element (threads 128..255) of every token
// of the next batch while the current batch is computed, so a batch costs one
// memory round trip rather than one per token.  Packed sequences read their
// bounds from cu_seqlens on the device.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int TB = 8;  // tokens per staged batch

template <typename InT, bool RAW>
__global__ __launch_bounds__(256) void prefill_recurrent_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const InT* __restrict__ beta, const float* __restrict__ log_alpha,
    const int32_t* __restrict__ cu_seqlens, int64_t T, int H,
    const StateRefs st, float* __restrict__ o,  // the final state may alias the initial one
    int64_t max_len)
{
    // double-buffered batches: [buffer][token][element]
    __shared__ __attribute__((aligned(16))) float sa[2][TB][kDim], sv[2][TB][kDim],
        sk[2][TB][kDim], sq[2][TB][kDim];
    __shared__ float sb[2][TB];
    const int64_t unit = blockIdx.x;  // n * H + h
    const int64_t n = unit / H;
    const int h = static_cast<int>(unit - n * H);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int rg = lane >> 3;
    const int row0 = 16 * rg;
    const int col = wave * 32 + (lane & 7) * 4;

    int64_t first, len;
    if (cu_seqlens) {
        first = cu_seqlens[n];
        len = static_cast<int64_t>(cu_seqlens[n + 1]) - first;
    } else {
        first = n * T;
        len = T;
    }
    if (max_len > 0 && len > max_len) return;  // left to the chunked kernel

    // this thread's staged element.  The requests are plain loads with no
    // branch around them (tokens past the end re-read the batch's first
    // token, and every thread loads the four inputs of its element), and the
    // raw values are converted only at staging: a load under a condition, or
    // converted right away, is compiled to wait for its data on the spot.
    const int e = tid & (kDim - 1);
    const bool gate_value = tid < kDim;
    float xa[TB];
    InT xv[TB], xk[TB], xq[TB], xb;
    auto request = [&](int64_t t0) {
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int64_t tt = t0 + t < len ? t0 + t : t0;
            const int64_t vec = ((first + tt) * H + h) * kDim;
            xa[t] = log_alpha[vec + e];
            xv[t] = v[vec + e];
            xk[t] = k[vec + e];
            xq[t] = q[vec + e];
        }
        const int64_t tb = t0 + (tid & (TB - 1));
        xb = beta[(first + (tb < len ? tb : t0)) * H + h];
    };
    auto stage = [&](int buf, int64_t t0) {
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t0 + t < len) {
                if (gate_value) {
                    sa[buf][t][e] = RAW ? alpha_from_logit(xa[t]) : exp_gate(xa[t]);
                    sv[buf][t][e] = widen(xv[t]);
                } else {
                    sk[buf][t][e] = widen(xk[t]);
                    sq[buf][t][e] = widen(xq[t]);
                }
            }
        }
        if (tid < TB && t0 + tid < len) sb[buf][tid] = RAW ? sigmoid_gate(widen(xb)) : widen(xb);
    };

    if (len > 0) request(0);   // (its loads read token 0, which an empty sequence does not have)
    float4 s[16];
    if (const float* S0 = init_state_of(st, n, h, H)) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
            s[m] = *reinterpret_cast<const float4*>(S0 + (row0 + m) * kDim + col);
    } else {
#pragma unroll
        for (int m = 0; m < 16; ++m) s[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // One barrier per batch: a wave writes a buffer again two batches later,
    // after the barrier that every wave reaches only once done with it.
    int buf = 0;
    for (int64_t t0 = 0; t0 < len; t0 += TB, buf ^= 1) {
        stage(buf, t0);
        __syncthreads();
        if (t0 + TB < len) request(t0 + TB);
        const int nb = static_cast<int>(len - t0 < TB ? len - t0 : TB);
        for (int t = 0; t < nb; ++t) {
            const float4 vt = *reinterpret_cast<const float4*>(&sv[buf][t][col]);
            const float4 ot = token_update<InT, RAW>(s, &sa[buf][t][row0], &sk[buf][t][row0],
                                                     &sq[buf][t][row0], sb[buf][t], vt);
            if (rg == 0)
                *reinterpret_cast<float4*>(o + ((first + t0 + t) * H + h) * kDim + col) = ot;
        }
    }

    if (float* S1 = final_state_of(st, n, h, H)) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
            *reinterpret_cast<float4*>(S1 + (row0 + m) * kDim + col) = s[m];
    }
}

}  // namespace

hipError_t launch_prefill_recurrent(const void* q, const void* k, const void* v,
                                    const void* beta, const float* log_alpha,
                                    const int32_t* cu_seqlens, int64_t n_seq, int64_t T,
                                    int64_t H, const StateRefs& st, float* o, bool bf16,
                                    bool raw, int64_t max_len, hipStream_t stream)
{
    const int64_t units = n_seq * H;
    if (units <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(units)), block(256);
    const int h = static_cast<int>(H);
    auto go = [&](auto kernel, auto tag) {
        using E = decltype(tag);
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, static_cast<const E*>(q),
                           static_cast<const E*>(k), static_cast<const E*>(v),
                           static_cast<const E*>(beta), log_alpha, cu_seqlens, T, h, st, o,
                           max_len);
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
