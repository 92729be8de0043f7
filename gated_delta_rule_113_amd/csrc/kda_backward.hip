// Backward pass of the KDA recurrence (gradients for training), token by token
// with the state and its gradient held in registers.
//
// Forward, per token (decay first, then erase and write; read-out from the
// updated state):
//     S' = Diag(a) S_{t-1},  p = S'^T k,  u = b (v - p),  S_t = S' + k u^T,  o = S_t^T q
// with a = exp(log_alpha_t).  Given dO (the gradient of the loss in every o_t)
// and dS_T (in the final state), the chain rule taken through one token in
// reverse, with G the gradient in S_t (everything after token t included):
//     G  += q dO^T                       (o = S_t^T q)
//     dq  = S_t dO = S' dO + k (u . dO)
//     du  = G^T k,   dv = b du,   db = du . (v - p),   dp = -b du
//     dk  = G u + S' dp                  (k writes through u and reads through p)
//     G'  = G + k dp^T                   (the gradient in S')
//     d log a_i = sum_j G'_ij S'_ij      (S' = Diag(a) S_{t-1})
//     G  <- Diag(a) G'                   (the gradient in S_{t-1})
// and after the first token G is the gradient in the initial state.
//
// The reverse sweep needs S_{t-1} at every token, which cannot be recovered
// from S_t (Diag(a) is not stably invertible when a channel forgets fast).
// Each workgroup therefore first runs the recurrence forward and stores the
// state every `cb` tokens (a checkpoint, 64 KiB per head) in a workspace;
// the reverse sweep then takes the blocks of cb tokens last to first, loads
// the block's checkpoint into registers and, for each token of the block from
// the last, recomputes the state up to that token from the checkpoint.  This
// costs (cb - 1) / 2 extra token updates per token and moves 128 KiB / cb per
// head-token through the workspace.
//
// Mapping: one workgroup of 256 threads per (sequence, head), with the lane
// mapping of the other token-by-token kernels (wave w: state columns
// 32w .. 32w+31; lane l: rows 16*(l >> 3) .. +15 of columns 32w + 4*(l & 7)
// .. +3), for the state, its checkpoint and its gradient (192 registers).
// Column sums (p, du) stay inside a wave; row sums (dq, dk, d log a) are
// summed over the wave's 8 column groups with DPP and over the 4 waves
// through LDS, double-buffered by token parity so that one barrier per token
// suffices.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int64_t SS = int64_t(kDim) * kDim;  // floats per state

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* beta;
    const float* log_alpha;
    const float* d_o;
    const int32_t* cu_seqlens;  // NULL: dense, sequence n = rows n*T .. n*T+T-1
    int64_t T;
    int H;
    const float* s0;    // [n_seq, H, 128, 128] or NULL (zeros)
    const float* d_sT;  // [n_seq, H, 128, 128] or NULL (zeros)
    float* dq;
    float* dk;
    float* dv;
    float* dbeta;
    float* dla;
    float* ds0;         // [n_seq, H, 128, 128] or NULL (not written)
    float* ckpt;        // workspace: n_slots * H states
    int cb;             // checkpoint interval, 1 <= cb <= kMaxBackwardBlock
    int64_t n_slots;
};

// Sum over the 8 lanes that differ in lane bits 0..2 (the 8 column groups of
// a row group): quad swaps by 1 and 2, then the mirror within each 8 lanes.
__device__ __forceinline__ float sum_cols8(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    return x;
}

__device__ __forceinline__ float dot4(float4 a, float4 b)
{
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// S' = Diag(a) S on the lane's share; returns p = S'^T k for its 4 columns
// (summed over all 128 rows).
__device__ __forceinline__ float4 decay_and_read(float4 (&s)[16], const float* a, const float* k)
{
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
        const float4 a4 = *reinterpret_cast<const float4*>(a + 4 * m4);
        const float4 k4 = *reinterpret_cast<const float4*>(k + 4 * m4);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
        const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * m4 + i;
            s[m].x *= av[i]; s[m].y *= av[i]; s[m].z *= av[i]; s[m].w *= av[i];
            p0 += kv[i] * s[m].x; p1 += kv[i] * s[m].y; p2 += kv[i] * s[m].z; p3 += kv[i] * s[m].w;
        }
    }
    return make_float4(xor_sum_rows(p0), xor_sum_rows(p1), xor_sum_rows(p2), xor_sum_rows(p3));
}

// One token forward on the lane's share: S <- Diag(a) S + k u^T, u = b (v - p).
__device__ __forceinline__ void forward_token(float4 (&s)[16], const float* a, const float* k,
                                              float bt, float4 vt)
{
    const float4 p = decay_and_read(s, a, k);
    const float4 u = make_float4(bt * (vt.x - p.x), bt * (vt.y - p.y), bt * (vt.z - p.z),
                                 bt * (vt.w - p.w));
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
        const float4 k4 = *reinterpret_cast<const float4*>(k + 4 * m4);
        const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * m4 + i;
            s[m].x += kv[i] * u.x; s[m].y += kv[i] * u.y; s[m].z += kv[i] * u.z; s[m].w += kv[i] * u.w;
        }
    }
}

template <typename InT>
__global__ __launch_bounds__(256, 1) void backward_kernel(const BwdArgs a)
{
    // one block of cb tokens staged: gates (as factors), keys, queries,
    // values, output gradients; beta
    __shared__ __attribute__((aligned(16))) float sa[kMaxBackwardBlock][kDim],
        sk[kMaxBackwardBlock][kDim], sq[kMaxBackwardBlock][kDim], sv[kMaxBackwardBlock][kDim],
        sdo[kMaxBackwardBlock][kDim];
    __shared__ float sb[kMaxBackwardBlock];
    // per-wave row sums [token parity][dq, dk, d log a][wave][row] and
    // scalars [token parity][u . dO, d beta][wave]
    __shared__ __attribute__((aligned(16))) float red[2][3][4][kDim];
    __shared__ float sred[2][2][4];

    const InT* Q = static_cast<const InT*>(a.q);
    const InT* K = static_cast<const InT*>(a.k);
    const InT* V = static_cast<const InT*>(a.v);
    const InT* B = static_cast<const InT*>(a.beta);
    const int H = a.H;
    const int64_t unit = blockIdx.x;  // n * H + h
    const int64_t n = unit / H;
    const int h = static_cast<int>(unit - n * H);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int rg = lane >> 3;
    const int row0 = 16 * rg;
    const int col = 32 * wave + 4 * (lane & 7);
    const int cb = a.cb;

    int64_t first, len, slot0;
    if (a.cu_seqlens) {
        first = a.cu_seqlens[n];
        len = static_cast<int64_t>(a.cu_seqlens[n + 1]) - first;
        // floor(first / cb) + n: sequences get disjoint runs of slots
        slot0 = first / cb + n;
    } else {
        first = n * a.T;
        len = a.T;
        slot0 = n * ((a.T + cb - 1) / cb);
    }
    if (len < 0 || first < 0) return;  // malformed cu_seqlens
    const int64_t nb = (len + cb - 1) / cb;
    if (slot0 + nb > a.n_slots) return;  // malformed cu_seqlens: stay inside the workspace
    auto ckpt_of = [&](int64_t b) { return a.ckpt + ((slot0 + b) * H + h) * SS; };

    // Stage tokens t0 .. t0+nt-1 of the sequence: threads 0..127 take one
    // gate and one value element (and with `all` one output-gradient
    // element) of each token, threads 128..255 one key (and query) element.
    const int e = tid & (kDim - 1);
    auto stage = [&](int64_t t0, int nt, bool all) {
#pragma unroll
        for (int t = 0; t < kMaxBackwardBlock; ++t) {
            if (t < nt) {
                const int64_t vec = ((first + t0 + t) * H + h) * kDim + e;
                if (tid < kDim) {
                    sa[t][e] = exp_gate(a.log_alpha[vec]);
                    sv[t][e] = widen(V[vec]);
                    if (all) sdo[t][e] = a.d_o[vec];
                } else {
                    sk[t][e] = widen(K[vec]);
                    if (all) sq[t][e] = widen(Q[vec]);
                }
            }
        }
        if (tid < nt) sb[tid] = widen(B[(first + t0 + tid) * H + h]);
    };
    auto load_state = [&](float4 (&x)[16], const float* src) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
            x[m] = src ? *reinterpret_cast<const float4*>(src + (row0 + m) * kDim + col)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    auto store_state = [&](const float4 (&x)[16], float* dst) {
#pragma unroll
        for (int m = 0; m < 16; ++m) *reinterpret_cast<float4*>(dst + (row0 + m) * kDim + col) = x[m];
    };

    // ---- forward sweep: a checkpoint at the start of every block
    float4 s[16];
    load_state(s, a.s0 ? a.s0 + unit * SS : nullptr);
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t t0 = b * cb;
        const int nt = static_cast<int>(len - t0 < cb ? len - t0 : cb);
        store_state(s, ckpt_of(b));
        stage(t0, nt, false);
        __syncthreads();
        for (int t = 0; t < nt; ++t)
            forward_token(s, &sa[t][row0], &sk[t][row0], sb[t],
                          *reinterpret_cast<const float4*>(&sv[t][col]));
        __syncthreads();  // the next block's staging overwrites this one
    }

    // ---- reverse sweep
    float4 G[16];
    load_state(G, a.d_sT ? a.d_sT + unit * SS : nullptr);
    int par = 0;
    for (int64_t b = nb - 1; b >= 0; --b) {
        const int64_t t0 = b * cb;
        const int nt = static_cast<int>(len - t0 < cb ? len - t0 : cb);
        float4 ck[16];
        load_state(ck, ckpt_of(b));
        stage(t0, nt, true);
        __syncthreads();
        for (int tt = nt - 1; tt >= 0; --tt) {
#pragma unroll
            for (int m = 0; m < 16; ++m) s[m] = ck[m];
            for (int t = 0; t < tt; ++t)
                forward_token(s, &sa[t][row0], &sk[t][row0], sb[t],
                              *reinterpret_cast<const float4*>(&sv[t][col]));
            // s = S_{t-1} -> S', and u
            const float* ar = &sa[tt][row0];
            const float* kr = &sk[tt][row0];
            const float* qr = &sq[tt][row0];
            const float bt = sb[tt];
            const float4 vt = *reinterpret_cast<const float4*>(&sv[tt][col]);
            const float4 dot = *reinterpret_cast<const float4*>(&sdo[tt][col]);
            const float4 p = decay_and_read(s, ar, kr);
            const float4 vp = make_float4(vt.x - p.x, vt.y - p.y, vt.z - p.z, vt.w - p.w);
            const float4 u = make_float4(bt * vp.x, bt * vp.y, bt * vp.z, bt * vp.w);

            // G += q dO^T;  du = G^T k
            float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
                const float4 q4 = *reinterpret_cast<const float4*>(qr + 4 * m4);
                const float4 k4 = *reinterpret_cast<const float4*>(kr + 4 * m4);
                const float qv[4] = {q4.x, q4.y, q4.z, q4.w};
                const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = 4 * m4 + i;
                    G[m].x += qv[i] * dot.x; G[m].y += qv[i] * dot.y;
                    G[m].z += qv[i] * dot.z; G[m].w += qv[i] * dot.w;
                    d0 += kv[i] * G[m].x; d1 += kv[i] * G[m].y; d2 += kv[i] * G[m].z; d3 += kv[i] * G[m].w;
                }
            }
            const float4 du = make_float4(xor_sum_rows(d0), xor_sum_rows(d1), xor_sum_rows(d2),
                                          xor_sum_rows(d3));
            const float4 dp = make_float4(-bt * du.x, -bt * du.y, -bt * du.z, -bt * du.w);

            // row sums over the lane's 4 columns, then over the wave's 32:
            // dq part S' dO, dk = G u + S' dp; then G' = G + k dp^T and
            // d log a = rowsum(G' .* S'); G <- Diag(a) G'
            float* rq = &red[par][0][wave][row0];
            float* rk = &red[par][1][wave][row0];
            float* rl = &red[par][2][wave][row0];
            float r[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) r[m] = sum_cols8(dot4(s[m], dot));
            if ((lane & 7) == 0) {
#pragma unroll
                for (int m4 = 0; m4 < 4; ++m4)
                    *reinterpret_cast<float4*>(rq + 4 * m4) =
                        make_float4(r[4 * m4], r[4 * m4 + 1], r[4 * m4 + 2], r[4 * m4 + 3]);
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) r[m] = sum_cols8(dot4(G[m], u) + dot4(s[m], dp));
            if ((lane & 7) == 0) {
#pragma unroll
                for (int m4 = 0; m4 < 4; ++m4)
                    *reinterpret_cast<float4*>(rk + 4 * m4) =
                        make_float4(r[4 * m4], r[4 * m4 + 1], r[4 * m4 + 2], r[4 * m4 + 3]);
            }
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
                const float4 a4 = *reinterpret_cast<const float4*>(ar + 4 * m4);
                const float4 k4 = *reinterpret_cast<const float4*>(kr + 4 * m4);
                const float av[4] = {a4.x, a4.y, a4.z, a4.w};
                const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = 4 * m4 + i;
                    G[m].x += kv[i] * dp.x; G[m].y += kv[i] * dp.y;
                    G[m].z += kv[i] * dp.z; G[m].w += kv[i] * dp.w;
                    r[m] = sum_cols8(dot4(G[m], s[m]));
                    G[m].x *= av[i]; G[m].y *= av[i]; G[m].z *= av[i]; G[m].w *= av[i];
                }
            }
            if ((lane & 7) == 0) {
#pragma unroll
                for (int m4 = 0; m4 < 4; ++m4)
                    *reinterpret_cast<float4*>(rl + 4 * m4) =
                        make_float4(r[4 * m4], r[4 * m4 + 1], r[4 * m4 + 2], r[4 * m4 + 3]);
            }
            // scalars over the wave's 32 columns (identical in every row group)
            const float x1 = sum_cols8(dot4(u, dot));
            const float x2 = sum_cols8(dot4(du, vp));
            if (lane == 0) {
                sred[par][0][wave] = x1;
                sred[par][1][wave] = x2;
            }
            const int64_t row = first + t0 + tt;
            const int64_t vec = (row * H + h) * kDim;
            if (rg == 0)
                *reinterpret_cast<float4*>(a.dv + vec + col) =
                    make_float4(bt * du.x, bt * du.y, bt * du.z, bt * du.w);
            __syncthreads();
            if (tid < kDim) {
                const int i = tid;
                float gq = 0.f, gk = 0.f, gl = 0.f, ud = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    gq += red[par][0][w][i];
                    gk += red[par][1][w][i];
                    gl += red[par][2][w][i];
                    ud += sred[par][0][w];
                }
                a.dq[vec + i] = gq + sk[tt][i] * ud;
                a.dk[vec + i] = gk;
                a.dla[vec + i] = gl;
            } else if (tid == kDim) {
                a.dbeta[row * H + h] =
                    sred[par][1][0] + sred[par][1][1] + sred[par][1][2] + sred[par][1][3];
            }
            par ^= 1;
        }
        __syncthreads();  // the next block's staging overwrites this one
    }
    if (a.ds0) store_state(G, a.ds0 + unit * SS);
}

}  // namespace

hipError_t launch_backward(const void* q, const void* k, const void* v, const void* beta,
                           const float* log_alpha, const float* d_o, const int32_t* cu_seqlens,
                           int64_t n_seq, int64_t T, int64_t T_total, int64_t H,
                           const float* initial_state, const float* d_final_state, float* dq,
                           float* dk, float* dv, float* dbeta, float* dlog_alpha,
                           float* d_initial_state, bool bf16, hipStream_t stream)
{
    const int64_t units = n_seq * H;
    if (units <= 0) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    report("hipGetDevice", e);
    if (e != hipSuccess) return e;
    report("earlier HIP error (cleared)", hipGetLastError());

    BwdArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.log_alpha = log_alpha;
    a.d_o = d_o;
    a.cu_seqlens = cu_seqlens;
    a.T = T;
    a.H = static_cast<int>(H);
    a.s0 = initial_state;
    a.d_sT = d_final_state;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dbeta = dbeta;
    a.dla = dlog_alpha;
    a.ds0 = d_initial_state;

    // Checkpoint interval: the shortest (least recomputation) whose
    // workspace stays within kBackwardWorkspaceCap, else the longest.
    const int64_t rows = cu_seqlens ? T_total : n_seq * T;
    auto slots_for = [&](int64_t cb) {
        return cu_seqlens ? T_total / cb + n_seq : n_seq * ((T + cb - 1) / cb);
    };
    int64_t cb = kBackwardBlock;
    while (cb < kMaxBackwardBlock &&
           slots_for(cb) * H * SS * static_cast<int64_t>(sizeof(float)) > kBackwardWorkspaceCap)
        cb *= 2;
    a.cb = static_cast<int>(cb);
    a.n_slots = rows > 0 ? slots_for(cb) : 0;

    void* ws = nullptr;
    if (a.n_slots > 0) {
        const size_t bytes = static_cast<size_t>(a.n_slots) * H * SS * sizeof(float);
        hipMemPool_t pool = workspace_pool(dev);
        if (!pool) return hipErrorOutOfMemory;
        e = hipMallocFromPoolAsync(&ws, bytes, pool, stream);
        report("hipMallocFromPoolAsync", e);
        if (e != hipSuccess) return e;
        a.ckpt = static_cast<float*>(ws);
    }
    const dim3 grid(static_cast<unsigned>(units)), block(256);
    if (bf16) hipLaunchKernelGGL(backward_kernel<bf16_t>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(backward_kernel<float>, grid, block, 0, stream, a);
    e = hipGetLastError();
    report("backward launch", e);
    if (ws) {
        const hipError_t f = hipFreeAsync(ws, stream);
        report("hipFreeAsync", f);
        if (e == hipSuccess) e = f;
    }
    return e;
}

}  // namespace kda
