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
// state every cb = 8 tokens (a checkpoint, 64 KiB per head) in a workspace;
// the reverse sweep then takes the blocks of 8 tokens last to first, loads the
// block's checkpoint into registers, computes the state after the block's 4th
// token into LDS and, for each token of the block from the last, recomputes
// its entering state from the nearer of the two.  This costs 2 extra token
// updates per token on average and moves 16 KiB per head-token through the
// workspace (8 KiB written, 8 KiB read).
//
// Mapping: one workgroup of 512 threads per (sequence, head) (see Layout
// and BackwardLayout below): each lane holds 8 rows x 4 columns of the state,
// its block checkpoint and its gradient in registers.  Column sums (p, du)
// stay inside a wave (DPP row rotations and the gfx950 lane swaps); row sums
// (dq, dk, d log a) are summed over the wave's column groups with DPP and over
// the 8 waves through LDS, double-buffered by token parity so that one
// barrier per token suffices.  The next block's inputs and checkpoint are
// requested while the current block is computed.  The work is fp32 vector
// arithmetic, about 1000 instructions per wave and token; no matrix
// instruction is involved.
#include <algorithm>
#include <type_traits>

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
    int cb;             // checkpoint interval, 1 <= cb <= kBackwardBlock
    int64_t n_slots;
};

// Lane layout of the state, its checkpoint and its gradient: wave w owns the
// 4*CG columns 4*CG*w ..; lane l holds R consecutive rows R*(l / CG) .. of
// the 4 columns 4*CG*w + 4*(l % CG) ..  (CG column groups times 128 / R row
// groups = 64 lanes).
template <int R_, int CG_>
struct Layout {
    static constexpr int R = R_;              // rows per lane
    static constexpr int CG = CG_;            // column groups per wave
    static constexpr int RG = kDim / R_;      // row groups per wave
    static constexpr int NW = kDim / (4 * CG_);  // waves
    static constexpr int NT = 64 * NW;        // threads
    static_assert(RG * CG == 64, "a wave is 64 lanes");
};

// 8 rows x 4 columns per lane, 16 columns per wave, 8 waves (512 threads):
// two waves per SIMD for one (sequence, head), and a share of 32 registers
// per matrix, small enough for the checkpoint, the state and its gradient to
// stay in registers together.  (16 x 4 per lane with 4 waves runs one wave
// per SIMD and is about 8% slower; 4 x 4 with 16 waves spends more on the
// column sums and is slower still.)
using BackwardLayout = Layout<8, 4>;

// x plus x from another lane (DPP control C).  Every source lane of the
// patterns used here is valid, so bound_ctrl does not change the result; it
// lets the compiler fold the lane move into the add.
template <int C>
__device__ __forceinline__ float dpp_add_c(float x)
{
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), C, 0xF, 0xF, true));
}

// Sum over the CG column groups of a row group (lane bits below log2 CG).
template <int CG>
__device__ __forceinline__ float row_sum(float x)
{
    x = dpp_add_c<0xB1>(x);                    // lane ^ 1 (quad permutation)
    if (CG >= 4) x = dpp_add_c<0x4E>(x);       // lane ^ 2
    if (CG >= 8) x = dpp_add_c<0x141>(x);      // the other quad of 8 (half-row mirror)
    return x;
}

// Sum over the row groups of a column group (lane bits from log2 CG up):
// rotations within each 16-lane row, then the gfx950 lane swaps across rows
// 16 and 32 apart.
template <int CG>
__device__ __forceinline__ float col_sum(float x)
{
    if (CG <= 1) x = dpp_add_c<0x121>(x);      // row_ror 1
    if (CG <= 2) x = dpp_add_c<0x122>(x);      // row_ror 2
    if (CG <= 4) x = dpp_add_c<0x124>(x);      // row_ror 4
    if (CG <= 8) x = dpp_add_c<0x128>(x);      // row_ror 8
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

// Raw storage bits of one input element, and their value.
__device__ __forceinline__ uint32_t raw_bits(const bf16_t* p) { return p->bits; }
__device__ __forceinline__ uint32_t raw_bits(const float* p) { return __float_as_uint(*p); }
template <typename InT>
__device__ __forceinline__ float from_bits(uint32_t x)
{
    return std::is_same<InT, bf16_t>::value ? __uint_as_float(x << 16) : __uint_as_float(x);
}

__device__ __forceinline__ float dot4(float4 a, float4 b)
{
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// S' = Diag(a) S on the lane's share; returns p = S'^T k for its 4 columns
// (summed over all 128 rows).  a, k: the lane's R rows in LDS.
template <class Ly>
__device__ __forceinline__ float4 decay_and_read(float4 (&s)[Ly::R], const float* a, const float* k)
{
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int m4 = 0; m4 < Ly::R / 4; ++m4) {
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
    return make_float4(col_sum<Ly::CG>(p0), col_sum<Ly::CG>(p1), col_sum<Ly::CG>(p2),
                       col_sum<Ly::CG>(p3));
}

// One token forward on the lane's share: S <- Diag(a) S + k u^T, u = b (v - p).
template <class Ly>
__device__ __forceinline__ void forward_token(float4 (&s)[Ly::R], const float* a, const float* k,
                                              float bt, float4 vt)
{
    const float4 p = decay_and_read<Ly>(s, a, k);
    const float4 u = make_float4(bt * (vt.x - p.x), bt * (vt.y - p.y), bt * (vt.z - p.z),
                                 bt * (vt.w - p.w));
#pragma unroll
    for (int m4 = 0; m4 < Ly::R / 4; ++m4) {
        const float4 k4 = *reinterpret_cast<const float4*>(k + 4 * m4);
        const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * m4 + i;
            s[m].x += kv[i] * u.x; s[m].y += kv[i] * u.y; s[m].z += kv[i] * u.z; s[m].w += kv[i] * u.w;
        }
    }
}

// Barrier for LDS traffic only: each wave's LDS reads and writes complete
// before it; its global stores stay in flight (a __syncthreads() would also
// wait for those).  The memory clobber keeps the compiler from moving memory
// accesses across it.  Global memory is never shared between the waves of a
// workgroup here (each lane reads back only the checkpoints it wrote).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename InT, class Ly>
__global__ __launch_bounds__(Ly::NT, 1) void backward_kernel(const BwdArgs a)
{
    constexpr int R = Ly::R, NW = Ly::NW;
    static_assert(Ly::NT >= 3 * kDim, "staging takes three groups of 128 threads");
    constexpr int TB = kBackwardBlock;
    constexpr int MID = TB / 2;  // the state after this many tokens of a block is kept in LDS
    // blocks of cb tokens staged, double-buffered: gates (as factors), keys,
    // queries, values, output gradients; beta
    __shared__ __attribute__((aligned(16))) float sa[2][TB][kDim], sk[2][TB][kDim],
        sq[2][TB][kDim], sv[2][TB][kDim], sdo[2][TB][kDim];
    __shared__ float sb[2][TB];
    // per-wave row sums [token parity][dq, dk, d log a][wave][row] and
    // scalars [token parity][u . dO, d beta][wave]
    __shared__ __attribute__((aligned(16))) float red[2][3][NW][kDim];
    __shared__ float sred[2][2][NW];
    // the state after the first MID tokens of the current block, each thread's
    // share in its own slots (written and read by the same thread only)
    __shared__ float4 smid[Ly::R][Ly::NT];

    const InT* Q = static_cast<const InT*>(a.q);
    const InT* K = static_cast<const InT*>(a.k);
    const InT* V = static_cast<const InT*>(a.v);
    const InT* B = static_cast<const InT*>(a.beta);
    const int H = a.H;
    const int64_t blk = blockIdx.x;
    const int64_t n = blk / H;
    const int h = static_cast<int>(blk - n * H);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int cg = lane % Ly::CG;
    const int rg = lane / Ly::CG;
    const int row0 = R * rg;
    const int col = 4 * Ly::CG * wave + 4 * cg;
    const int cb = a.cb;

    int64_t first, len, slot0;
    const int64_t unit = n * H + h;
    const float* s0p = a.s0 ? a.s0 + unit * SS : nullptr;     // entering state (NULL: zeros)
    const float* dsTp = a.d_sT ? a.d_sT + unit * SS : nullptr; // gradient in the leaving state
    float* ds0p = a.ds0 ? a.ds0 + unit * SS : nullptr;        // gradient in the entering state
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
    auto block_len = [&](int64_t b) { return static_cast<int>(len - b * cb < cb ? len - b * cb : cb); };

    // Inputs of a block, one element of a token's vector per thread: threads
    // 0..127 the gate and the value, 128..255 the key and the query,
    // 256..383 (with `all`) the output gradient; threads below cb beta.  They
    // are requested one block ahead as raw bits (so no instruction waits for
    // the loads) and widened when written to the LDS buffer of their block,
    // just before it is used.  `role` is uniform within a wave.
    const int e = tid & (kDim - 1);
    const int role = __builtin_amdgcn_readfirstlane(tid >> 7);
    uint32_t x0[TB], x1[TB], xb = 0;
    auto request = [&](int64_t b, bool all) {
        const int nt = block_len(b);
        const int64_t v0 = ((first + b * cb) * H + h) * kDim + e;
        const int64_t step = static_cast<int64_t>(H) * kDim;
        if (role == 0) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
                if (t < nt) {
                    x0[t] = __float_as_uint(a.log_alpha[v0 + t * step]);
                    x1[t] = raw_bits(V + v0 + t * step);
                }
        } else if (role == 1) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
                if (t < nt) {
                    x0[t] = raw_bits(K + v0 + t * step);
                    x1[t] = raw_bits(Q + v0 + t * step);
                }
        } else if (role == 2 && all) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
                if (t < nt) x0[t] = __float_as_uint(a.d_o[v0 + t * step]);
        }
        if (tid < nt) xb = raw_bits(B + (first + b * cb + tid) * H + h);
    };
    auto stage = [&](int buf, int nt, bool all) {
        if (role == 0) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
                if (t < nt) {
                    sa[buf][t][e] = exp_gate(__uint_as_float(x0[t]));
                    sv[buf][t][e] = from_bits<InT>(x1[t]);
                }
        } else if (role == 1) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
                if (t < nt) {
                    sk[buf][t][e] = from_bits<InT>(x0[t]);
                    sq[buf][t][e] = from_bits<InT>(x1[t]);
                }
        } else if (role == 2 && all) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
                if (t < nt) sdo[buf][t][e] = __uint_as_float(x0[t]);
        }
        if (tid < nt) sb[buf][tid] = from_bits<InT>(xb);
    };
    auto load_state = [&](float4 (&x)[R], const float* src) {
#pragma unroll
        for (int m = 0; m < R; ++m)
            x[m] = src ? *reinterpret_cast<const float4*>(src + (row0 + m) * kDim + col)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    auto store_state = [&](const float4 (&x)[R], float* dst) {
#pragma unroll
        for (int m = 0; m < R; ++m) *reinterpret_cast<float4*>(dst + (row0 + m) * kDim + col) = x[m];
    };
    // row sums of the R values of every lane over the whole wave, written to
    // this wave's slot of the LDS partial sums
    auto put_rows = [&](float (&r)[R], float* dst) {
#pragma unroll
        for (int m = 0; m < R; ++m) r[m] = row_sum<Ly::CG>(r[m]);
        if (cg == 0) {
#pragma unroll
            for (int m4 = 0; m4 < R / 4; ++m4)
                *reinterpret_cast<float4*>(dst + 4 * m4) =
                    make_float4(r[4 * m4], r[4 * m4 + 1], r[4 * m4 + 2], r[4 * m4 + 3]);
        }
    };
    // A buffer is written again two blocks after it was read; every wave has
    // passed the barrier of the block in between by then.

    // ---- forward sweep: a checkpoint at the start of every block
    float4 s[R];
    load_state(s, s0p);
    if (nb > 0) request(0, false);
    for (int64_t b = 0; b < nb; ++b) {
        const int buf = static_cast<int>(b & 1);
        const int nt = block_len(b);
        store_state(s, ckpt_of(b));
        stage(buf, nt, false);
        lds_barrier();
        if (b + 1 < nb) request(b + 1, false);
        for (int t = 0; t < nt; ++t)
            forward_token<Ly>(s, &sa[buf][t][row0], &sk[buf][t][row0], sb[buf][t],
                              *reinterpret_cast<const float4*>(&sv[buf][t][col]));
    }

    // ---- reverse sweep, blocks last to first
    float4 G[R], ck[R];
    load_state(G, dsTp);
    if (nb > 0) {
        request(nb - 1, true);
        load_state(ck, ckpt_of(nb - 1));
    }
    lds_barrier();  // the forward sweep's last block is no longer read
    int par = 0;
    for (int64_t b = nb - 1; b >= 0; --b) {
        const int buf = static_cast<int>(b & 1);
        const int nt = block_len(b);
        const int64_t t0 = b * cb;
        stage(buf, nt, true);
        lds_barrier();
        float4 ckn[R];
        if (b > 0) {
            request(b - 1, true);
            load_state(ckn, ckpt_of(b - 1));
        }
        // the state after MID tokens: the later tokens of the block are
        // recomputed from it rather than from the checkpoint
        const bool use_mid = nt > MID;
        if (use_mid) {
#pragma unroll
            for (int m = 0; m < R; ++m) s[m] = ck[m];
            for (int t = 0; t < MID; ++t)
                forward_token<Ly>(s, &sa[buf][t][row0], &sk[buf][t][row0], sb[buf][t],
                                  *reinterpret_cast<const float4*>(&sv[buf][t][col]));
#pragma unroll
            for (int m = 0; m < R; ++m) smid[m][tid] = s[m];
        }
        for (int tt = nt - 1; tt >= 0; --tt) {
            int t = 0;
            if (use_mid && tt >= MID) {
                t = MID;
#pragma unroll
                for (int m = 0; m < R; ++m) s[m] = smid[m][tid];
            } else {
#pragma unroll
                for (int m = 0; m < R; ++m) s[m] = ck[m];
            }
            for (; t < tt; ++t)
                forward_token<Ly>(s, &sa[buf][t][row0], &sk[buf][t][row0], sb[buf][t],
                                  *reinterpret_cast<const float4*>(&sv[buf][t][col]));
            // s = S_{t-1} -> S', and u
            const float* ar = &sa[buf][tt][row0];
            const float* kr = &sk[buf][tt][row0];
            const float* qr = &sq[buf][tt][row0];
            const float bt = sb[buf][tt];
            const float4 vt = *reinterpret_cast<const float4*>(&sv[buf][tt][col]);
            const float4 dot = *reinterpret_cast<const float4*>(&sdo[buf][tt][col]);
            const float4 p = decay_and_read<Ly>(s, ar, kr);
            const float4 vp = make_float4(vt.x - p.x, vt.y - p.y, vt.z - p.z, vt.w - p.w);
            const float4 u = make_float4(bt * vp.x, bt * vp.y, bt * vp.z, bt * vp.w);

            // G += q dO^T;  du = G^T k
            float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
            for (int m4 = 0; m4 < R / 4; ++m4) {
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
            const float4 du = make_float4(col_sum<Ly::CG>(d0), col_sum<Ly::CG>(d1),
                                          col_sum<Ly::CG>(d2), col_sum<Ly::CG>(d3));
            const float4 dp = make_float4(-bt * du.x, -bt * du.y, -bt * du.z, -bt * du.w);

            // row sums over the lane's 4 columns, then over the wave's: the dq
            // part S' dO; dk = G u + S' dp; then G' = G + k dp^T and
            // d log a = rowsum(G' .* S'); G <- Diag(a) G'
            float r[R];
#pragma unroll
            for (int m = 0; m < R; ++m) r[m] = dot4(s[m], dot);
            put_rows(r, &red[par][0][wave][row0]);
#pragma unroll
            for (int m = 0; m < R; ++m) r[m] = dot4(G[m], u) + dot4(s[m], dp);
            put_rows(r, &red[par][1][wave][row0]);
#pragma unroll
            for (int m4 = 0; m4 < R / 4; ++m4) {
                const float4 a4 = *reinterpret_cast<const float4*>(ar + 4 * m4);
                const float4 k4 = *reinterpret_cast<const float4*>(kr + 4 * m4);
                const float av[4] = {a4.x, a4.y, a4.z, a4.w};
                const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = 4 * m4 + i;
                    G[m].x += kv[i] * dp.x; G[m].y += kv[i] * dp.y;
                    G[m].z += kv[i] * dp.z; G[m].w += kv[i] * dp.w;
                    r[m] = dot4(G[m], s[m]);
                    G[m].x *= av[i]; G[m].y *= av[i]; G[m].z *= av[i]; G[m].w *= av[i];
                }
            }
            put_rows(r, &red[par][2][wave][row0]);
            // scalars over the wave's columns (identical in every row group)
            const float x1s = row_sum<Ly::CG>(dot4(u, dot));
            const float x2s = row_sum<Ly::CG>(dot4(du, vp));
            if (lane == 0) {
                sred[par][0][wave] = x1s;
                sred[par][1][wave] = x2s;
            }
            const int64_t row = first + t0 + tt;
            const int64_t vec = (row * H + h) * kDim;
            if (rg == 0)
                *reinterpret_cast<float4*>(a.dv + vec + col) =
                    make_float4(bt * du.x, bt * du.y, bt * du.z, bt * du.w);
            lds_barrier();
            // threads 0..127: dq and d log a of channel tid; 128..255: dk
            if (tid < 2 * kDim) {
                const int i = e;
                if (tid < kDim) {
                    float gq = 0.f, gl = 0.f, ud = 0.f;
#pragma unroll
                    for (int w = 0; w < NW; ++w) {
                        gq += red[par][0][w][i];
                        gl += red[par][2][w][i];
                        ud += sred[par][0][w];
                    }
                    a.dq[vec + i] = gq + sk[buf][tt][i] * ud;
                    a.dla[vec + i] = gl;
                } else {
                    float gk = 0.f, db = 0.f;
#pragma unroll
                    for (int w = 0; w < NW; ++w) {
                        gk += red[par][1][w][i];
                        db += sred[par][1][w];
                    }
                    a.dk[vec + i] = gk;
                    if (tid == kDim) a.dbeta[row * H + h] = db;
                }
            }
            par ^= 1;
        }
        if (b > 0) {
#pragma unroll
            for (int m = 0; m < R; ++m) ck[m] = ckn[m];
        }
    }
    if (ds0p) store_state(G, ds0p);
}

}  // namespace

hipError_t launch_backward(const void* q, const void* k, const void* v, const void* beta,
                           const float* log_alpha, const float* d_o, const int32_t* cu_seqlens,
                           int64_t n_seq, int64_t T, int64_t H, const float* initial_state,
                           const float* d_final_state, float* dq, float* dk, float* dv,
                           float* dbeta, float* dlog_alpha, float* d_initial_state, bool bf16,
                           const BackwardPlan& plan, void* ws, hipStream_t stream)
{
    const int64_t units = n_seq * H;
    if (units <= 0) return hipSuccess;
    if (plan.chunked)
        return launch_backward_chunked(q, k, v, beta, log_alpha, d_o, cu_seqlens, n_seq, T, H,
                                       initial_state, d_final_state, dq, dk, dv, dbeta, dlog_alpha,
                                       d_initial_state, plan.n_ids, ws, stream);
    hipError_t e = hipSuccess;

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
    a.cb = kBackwardBlock;
    a.n_slots = plan.n_slots;
    a.ckpt = static_cast<float*>(ws);

    // the token-by-token path serves fp32 inputs (bf16 ones take the chunked path)
    if (bf16) return hipErrorInvalidValue;
    using Ly = BackwardLayout;
    hipLaunchKernelGGL((backward_kernel<float, Ly>), dim3(static_cast<unsigned>(units)),
                       dim3(Ly::NT), 0, stream, a);
    e = hipGetLastError();
    report("backward launch", e);
    return e;
}

}  // namespace kda
