// Fused KDA decode step: one token per head, state streamed through HBM once.
//
// Per head (S is d_k x d_v = 128 x 128 fp32, rows = forgetting channels):
//   a = exp(log_alpha)                     channel-wise forgetting
//   S' = Diag(a) S                         (never stored)
//   p = S'^T k,  r = S'^T q                both reductions over the rows of S'
//   u = beta (v - p)                       the delta-rule correction
//   S <- S' + k u^T                        erase-then-write, stored in place
//   o = S^T q = r + (k . q) u
// The pages define the update ("Kimi K3 -- the architecture and infrastructure,
// explained", section "How the delta rule actually works", with the per-channel
// gate of section "Kimi Delta Attention: the load-bearing choice") and say the
// decode phase is bound by memory bandwidth, its cost per token constant; here
// each state byte is read once and written once per token.
//
// Mapping: one workgroup of 256 threads per head.  Wave w owns columns
// [32w, 32w+32).  Lane l owns columns 32w + 4*(l & 7) .. +3 and the 16
// consecutive rows 16*(l >> 3) .. +15: 16 float4 = 64 state values in
// registers.  Each load instruction of a wave covers 8 rows x 128 contiguous
// bytes.  The head's 128 gates, keys and queries are loaded once per
// workgroup (exp(log_alpha) and the bf16 widening done once) into LDS, from
// where every lane reads its 16 rows as float4.  The column
// reductions finish across the 8 row groups of a wave with lane shuffles.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

// A state row piece of 4 floats.  STREAM: with the nontemporal hint, for
// states that do not fit the last-level cache (then nothing is reused from it
// by the next step, and the hint keeps the stream from evicting what is);
// without it, a state that fits is read back from that cache at the next step.
typedef float nt4 __attribute__((ext_vector_type(4)));
template <bool STREAM>
__device__ __forceinline__ float4 state_ld(const float* p)
{
    if (STREAM) {
        const nt4 x = __builtin_nontemporal_load(reinterpret_cast<const nt4*>(p));
        return make_float4(x[0], x[1], x[2], x[3]);
    }
    return *reinterpret_cast<const float4*>(p);
}
typedef float nt2 __attribute__((ext_vector_type(2)));
template <bool STREAM>
__device__ __forceinline__ float2 state_ld2(const float* p)
{
    if (STREAM) {
        const nt2 x = __builtin_nontemporal_load(reinterpret_cast<const nt2*>(p));
        return make_float2(x[0], x[1]);
    }
    return *reinterpret_cast<const float2*>(p);
}
template <bool STREAM>
__device__ __forceinline__ void state_st(float* p, float4 t)
{
    if (STREAM) __builtin_nontemporal_store((nt4){t.x, t.y, t.z, t.w}, reinterpret_cast<nt4*>(p));
    else *reinterpret_cast<float4*>(p) = t;
}

template <typename InT, bool RAW, bool STREAM>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const InT* __restrict__ beta, const float* __restrict__ log_alpha,
    float* __restrict__ state, const int32_t* __restrict__ slots, int64_t n_pool, int H,
    float* __restrict__ o)
{
    __shared__ __attribute__((aligned(16))) float sa[kDim], sk[kDim], sq[kDim];
    const int64_t unit = blockIdx.x;  // n * H + h
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int rg = lane >> 3;
    const int row0 = 16 * rg;
    const int col = wave * 32 + (lane & 7) * 4;

    // the head's state: entry unit, or with slots entry (slots[n], h) of the
    // pool; a slot outside the pool skips the sequence (a whole-workgroup exit)
    int64_t e = unit;
    if (slots) {
        const int64_t n = unit / H;
        const int64_t sl = slots[n];
        if (sl < 0 || sl >= n_pool) return;
        e = sl * H + (unit - n * H);
    }
    float* S = state + e * (kDim * kDim);
    const int64_t vec = unit * kDim;

    // the per-head inputs come from memory not touched by earlier steps, so
    // they are requested first; the state usually streams from closer caches
    float x0, x1 = 0.f;
    if (tid < kDim) {
        x0 = log_alpha[vec + tid];
    } else {
        x0 = widen(k[vec + tid - kDim]);
        x1 = widen(q[vec + tid - kDim]);
    }
    const float4 vv = load4(v + vec + col);
    float bt = widen(beta[unit]);
    float4 s[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) s[m] = state_ld<STREAM>(S + (row0 + m) * kDim + col);

    if (tid < kDim) {
        sa[tid] = RAW ? alpha_from_logit(x0) : exp_gate(x0);
    } else {
        sk[tid - kDim] = x0;
        sq[tid - kDim] = x1;
    }
    __syncthreads();

    float a[16], kk[16], qq[16];
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
        const float4 a4 = *reinterpret_cast<const float4*>(sa + row0 + 4 * m4);
        const float4 k4 = *reinterpret_cast<const float4*>(sk + row0 + 4 * m4);
        const float4 q4 = *reinterpret_cast<const float4*>(sq + row0 + 4 * m4);
        a[4 * m4] = a4.x; a[4 * m4 + 1] = a4.y; a[4 * m4 + 2] = a4.z; a[4 * m4 + 3] = a4.w;
        kk[4 * m4] = k4.x; kk[4 * m4 + 1] = k4.y; kk[4 * m4 + 2] = k4.z; kk[4 * m4 + 3] = k4.w;
        qq[4 * m4] = q4.x; qq[4 * m4 + 1] = q4.y; qq[4 * m4 + 2] = q4.z; qq[4 * m4 + 3] = q4.w;
    }

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
        float4 t = s[m];
        t.x += kk[m] * u0; t.y += kk[m] * u1; t.z += kk[m] * u2; t.w += kk[m] * u3;
        state_st<STREAM>(S + (row0 + m) * kDim + col, t);
    }
}

constexpr float kLog2e = 1.4426950408889634f;

// The sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ float wave_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lane ^ 1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lane ^ 2
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)); // row_ror 4
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)); // row_ror 8
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

// K consecutive tokens of each sequence from its current state (speculative
// decoding: verify K draft tokens, then keep the accepted prefix).  The same
// per-token arithmetic and lane mapping as decode_step_kernel, with the state
// kept in registers across the tokens: it is read once, and written at most
// once -- in place, right after token n_commit[n] (n_commit[n] <= 0, or no
// n_commit at all, leaves it unchanged).  Every token's output is written.
// The K tokens' gates, keys, queries and write strengths are staged in LDS
// together before the state loads complete.
template <typename InT, int KM, bool STREAM>
__global__ __launch_bounds__(256) void decode_tokens_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const InT* __restrict__ beta, const float* __restrict__ log_alpha,
    float* __restrict__ state, const int32_t* __restrict__ n_commit, int K, int H,
    float* __restrict__ o)
{
    // KM >= K: token capacity of this instantiation (sizes the staging registers)
    __shared__ __attribute__((aligned(16))) float sa[KM][kDim], sk[KM][kDim], sq[KM][kDim], sb[KM];
    const int64_t unit = blockIdx.x;  // n * H + h
    const int64_t n = unit / H;
    const int h = static_cast<int>(unit - n * H);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int rg = lane >> 3;
    const int row0 = 16 * rg;
    const int col = wave * 32 + (lane & 7) * 4;
    float* S = state + unit * (kDim * kDim);
    const int commit = n_commit ? min(max(n_commit[n], 0), K) : 0;
    auto rowvec = [&](int t) { return ((n * K + t) * H + h) * kDim; };  // token t's [*, 128] row

    // all tokens' per-head inputs are requested first, then the state; both
    // are in flight together.  The loads have no branch around them (tokens
    // from K on re-read token 0; every thread loads the gate, key and query
    // element tid mod 128) and their raw values are converted only after all
    // of them are issued: a conditional load, or one converted right away,
    // is compiled to wait for its data on the spot.
    const int e = tid & (kDim - 1);
    float xa[KM];
    InT xk[KM], xq[KM], xb[KM];
#pragma unroll
    for (int t = 0; t < KM; ++t) {
        const int tt = t < K ? t : 0;
        const int64_t vec = rowvec(tt);
        xa[t] = log_alpha[vec + e];
        xk[t] = k[vec + e];
        xq[t] = q[vec + e];
        xb[t] = beta[(n * K + tt) * H + h];
    }
    float4 s[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
        s[m] = state_ld<STREAM>(S + (row0 + m) * kDim + col);
    auto vrow = [&](int t) { return v + rowvec(t) + col; };
    auto vraw = load4_raw(vrow(0));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < KM; ++t) {
        if (t < K) {
            if (tid < kDim) {
                sa[t][e] = exp_gate(xa[t]);
            } else {
                sk[t][e] = widen(xk[t]);
                sq[t][e] = widen(xq[t]);
            }
            if (tid == 0) sb[t] = widen(xb[t]);
        }
    }
    __syncthreads();

    for (int t = 0; t < K; ++t) {
        const float4 vt = widen4(vraw);
        vraw = load4_raw(vrow(t + 1 < K ? t + 1 : t));   // (the last token re-reads its own row)
        const float4 ot = token_update<InT, false>(s, &sa[t][row0], &sk[t][row0], &sq[t][row0], sb[t], vt);
        if (rg == 0) *reinterpret_cast<float4*>(o + rowvec(t) + col) = ot;
        if (t + 1 == commit) {
#pragma unroll
            for (int m = 0; m < 16; ++m) state_st<STREAM>(S + (row0 + m) * kDim + col, s[m]);
        }
    }
}

// Verify only (no commit) for K <= 4: the K tokens as one chunk of the
// blockwise form ("Kimi K3 -- the architecture and infrastructure,
// explained", section "Kimi Delta Attention: the load-bearing choice": the
// delta rule regrouped per block of tokens), in fp32 on the vector ALUs.
// With G_t the cumulative log2-decay of each channel over tokens 0..t and S
// the entering state:
//     A_ri = sum_c k_rc k_ic 2^(G_rc - G_ic) (i < r),  P_ri = sum_c q_rc k_ic 2^(G_rc - G_ic) (i <= r)
//     X_r = S^T (k_r (.) 2^G_r),   Y_r = S^T (q_r (.) 2^G_r)
//     U_r = b_r (v_r - X_r - sum_{i<r} A_ri U_i),   o_r = Y_r + sum_{i<=r} P_ri U_i
// (all exponents <= 0).  Per token a lane does 128 multiply-adds per 64
// state elements (X and Y) instead of the 256 of a state update and readout,
// and the state is only read, so it is streamed through registers in blocks
// of 4 rows instead of held: a lane needs few registers and every head of a
// decode batch can be resident at once (8 waves per SIMD), the loads of later
// blocks overlapping the arithmetic of earlier ones.  The pair sums grow as
// K^2, so longer drafts and commits keep the token-by-token kernel above.  Lane mapping: wave w owns columns 32w..32w+31,
// lane l the columns 32w + 2 (l & 15) .. +1 of the 32 rows 32 (l >> 4) .. +31
// (one load instruction of a wave covers 4 rows x 128 contiguous bytes).
template <typename InT, bool STREAM>
__global__ __launch_bounds__(256, 8) void decode_verify4_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const InT* __restrict__ beta, const float* __restrict__ log_alpha,
    const float* __restrict__ state, int K, int H, float* __restrict__ o)
{
    constexpr int KM = 4, NP = KM * (KM + 1) / 2, NB = 8;   // tokens, pairs, 4-row blocks per lane
    __shared__ __attribute__((aligned(16))) float sKt[KM][kDim], sQt[KM][kDim];
    __shared__ float pA[NP][2], pP[NP][2];
    const int64_t unit = blockIdx.x;  // n * H + h
    const int64_t n = unit / H;
    const int h = static_cast<int>(unit - n * H);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r0 = 32 * (lane >> 4);
    const int col = 32 * wave + 2 * (lane & 15);
    const float* S = state + unit * (kDim * kDim) + col;
    auto rowvec = [&](int t) { return ((n * K + t) * H + h) * kDim; };

    // inputs first (no branch around a load: tokens from K on re-read token 0),
    // then the first two blocks of the state
    const int e = tid & (kDim - 1);
    float xa[KM];
    InT xk[KM], xq[KM], xb[KM];
    decltype(load2_raw(v)) vr[KM];
#pragma unroll
    for (int t = 0; t < KM; ++t) {
        const int tt = t < K ? t : 0;
        const int64_t vec = rowvec(tt);
        xa[t] = log_alpha[vec + e];
        xk[t] = k[vec + e];
        xq[t] = q[vec + e];
        xb[t] = beta[(n * K + tt) * H + h];
        vr[t] = load2_raw(v + vec + col);
    }
    float2 blk[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) blk[b][i] = state_ld2<STREAM>(S + (r0 + 4 * b + i) * kDim);
    __builtin_amdgcn_sched_barrier(0);

    // per channel e: G, the decayed keys and queries (first half), the pairs'
    // terms of A and P (both halves, by parity)
    const int half = wave >> 1;
    float g[KM], kv[KM], qv[KM];
    {
        float run = 0.f;
#pragma unroll
        for (int t = 0; t < KM; ++t) {
            run += t < K ? xa[t] * kLog2e : 0.f;
            g[t] = run;
            kv[t] = widen(xk[t]);
            qv[t] = widen(xq[t]);
        }
    }
    if (half == 0) {
#pragma unroll
        for (int t = 0; t < KM; ++t) {
            if (t < K) {
                const float gm = __builtin_amdgcn_exp2f(g[t]);
                sKt[t][e] = kv[t] * gm;
                sQt[t][e] = qv[t] * gm;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < KM; ++r)
#pragma unroll
        for (int i = 0; i <= r; ++i) {
            const int p = r * (r + 1) / 2 + i;
            if (r < K && (p & 1) == half) {
                const float f = kv[i] * __builtin_amdgcn_exp2f(g[r] - g[i]);
                const float av = i < r ? wave_sum(kv[r] * f) : 0.f;
                const float pv = wave_sum(qv[r] * f);
                if (lane == 0) {
                    pA[p][wave & 1] = av;
                    pP[p][wave & 1] = pv;
                }
            }
        }
    __syncthreads();

    // ---- X_t and Y_t over the lane's 32 rows, block by block, two blocks in flight
    float2 X[KM], Y[KM];
#pragma unroll
    for (int t = 0; t < KM; ++t) X[t] = Y[t] = make_float2(0.f, 0.f);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float2 (&cur)[4] = blk[b & 1];
#pragma unroll
        for (int t = 0; t < KM; ++t) {
            if (t >= K) continue;
            const float4 k4 = *reinterpret_cast<const float4*>(&sKt[t][r0 + 4 * b]);
            const float4 q4 = *reinterpret_cast<const float4*>(&sQt[t][r0 + 4 * b]);
            const float kt[4] = {k4.x, k4.y, k4.z, k4.w}, qt[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                X[t].x += kt[i] * cur[i].x; X[t].y += kt[i] * cur[i].y;
                Y[t].x += qt[i] * cur[i].x; Y[t].y += qt[i] * cur[i].y;
            }
        }
        if (b + 2 < NB) {
#pragma unroll
            for (int i = 0; i < 4; ++i) cur[i] = state_ld2<STREAM>(S + (r0 + 4 * (b + 2) + i) * kDim);
        }
    }
    // sums over the four row quarters (lanes l, l ^ 16, l ^ 32, l ^ 48)
    auto quarters = [](float x) {
        const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
        const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
    };
    float2 U[KM];
#pragma unroll
    for (int r = 0; r < KM; ++r) {
        if (r >= K) continue;
        const float2 x = make_float2(quarters(X[r].x), quarters(X[r].y));
        const float2 y = make_float2(quarters(Y[r].x), quarters(Y[r].y));
        const float2 vt = widen2(vr[r]);
        float2 u = make_float2(vt.x - x.x, vt.y - x.y);
#pragma unroll
        for (int i = 0; i < r; ++i) {
            const int p = r * (r + 1) / 2 + i;
            const float a_ = pA[p][0] + pA[p][1];
            u.x -= a_ * U[i].x; u.y -= a_ * U[i].y;
        }
        const float br = widen(xb[r]);
        U[r] = make_float2(br * u.x, br * u.y);
        float2 ot = y;
#pragma unroll
        for (int i = 0; i <= r; ++i) {
            const int p = r * (r + 1) / 2 + i;
            const float p_ = pP[p][0] + pP[p][1];
            ot.x += p_ * U[i].x; ot.y += p_ * U[i].y;
        }
        if (r0 == 0) *reinterpret_cast<float2*>(o + rowvec(r) + col) = ot;
    }
}

}  // namespace

// Whether a call's states (64 KiB per head) exceed the 256 MB last-level
// cache: then its kernels stream them with the nontemporal hint.
static bool streams_state(int64_t units)
{
    constexpr int64_t kStreamBytes = int64_t(256) << 20;
    return units * static_cast<int64_t>(kDim * kDim * sizeof(float)) > kStreamBytes;
}

hipError_t launch_decode_tokens(const void* q, const void* k, const void* v, const void* beta,
                                const float* log_alpha, float* state, const int32_t* n_commit,
                                float* o, int64_t N, int64_t K, int64_t H, bool bf16,
                                hipStream_t stream)
{
    const int64_t units = N * H;
    if (units <= 0 || K <= 0) return hipSuccess;
    if (K > kMaxDraft) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(units)), block(256);
    auto go = [&](auto km, auto tag, auto str) {
        using T = decltype(tag);
        constexpr int KMV = decltype(km)::value;
        constexpr bool ST = decltype(str)::value;
        hipLaunchKernelGGL((decode_tokens_kernel<T, KMV, ST>), grid, block, 0, stream,
                           static_cast<const T*>(q), static_cast<const T*>(k),
                           static_cast<const T*>(v), static_cast<const T*>(beta), log_alpha,
                           state, n_commit, static_cast<int>(K), static_cast<int>(H), o);
    };
    auto verify4 = [&](auto tag, auto str) {
        using T = decltype(tag);
        constexpr bool ST = decltype(str)::value;
        hipLaunchKernelGGL((decode_verify4_kernel<T, ST>), grid, block, 0, stream, static_cast<const T*>(q),
                           static_cast<const T*>(k), static_cast<const T*>(v), static_cast<const T*>(beta),
                           log_alpha, state, static_cast<int>(K), static_cast<int>(H), o);
    };
    auto pick = [&](auto tag, auto str) {
        if (K <= 4 && !n_commit) verify4(tag, str);
        else if (K <= 4) go(std::integral_constant<int, 4>{}, tag, str);
        else if (K <= 8) go(std::integral_constant<int, 8>{}, tag, str);
        else go(std::integral_constant<int, 16>{}, tag, str);
    };
    const bool st = streams_state(units);
    if (bf16) st ? pick(bf16_t{}, std::true_type{}) : pick(bf16_t{}, std::false_type{});
    else st ? pick(0.f, std::true_type{}) : pick(0.f, std::false_type{});
    return hipGetLastError();
}

hipError_t launch_decode_step(const void* q, const void* k, const void* v, const void* beta,
                              const float* log_alpha, float* state, const int32_t* slots,
                              int64_t n_pool, float* o, int64_t units, int64_t H, bool bf16,
                              bool raw, hipStream_t stream)
{
    if (units <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(units)), block(256);
    auto go = [&](auto kernel, auto tag) {
        using T = decltype(tag);
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, static_cast<const T*>(q),
                           static_cast<const T*>(k), static_cast<const T*>(v),
                           static_cast<const T*>(beta), log_alpha, state, slots, n_pool,
                           static_cast<int>(H), o);
    };
    auto pick = [&](auto str) {
        constexpr bool ST = decltype(str)::value;
        if (bf16) {
            if (raw) go(decode_step_kernel<bf16_t, true, ST>, bf16_t{});
            else go(decode_step_kernel<bf16_t, false, ST>, bf16_t{});
        } else {
            if (raw) go(decode_step_kernel<float, true, ST>, 0.f);
            else go(decode_step_kernel<float, false, ST>, 0.f);
        }
    };
    if (streams_state(units)) pick(std::true_type{});
    else pick(std::false_type{});
    return hipGetLastError();
}

}  // namespace kda
