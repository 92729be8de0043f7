// Chunked backward pass of the KDA prefill on bf16 matrix cores.
//
// The forward (per head; S is d_k x d_v, rows = forgetting channels)
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t
// ("Kimi K3 -- the architecture and infrastructure, explained": section "How
// the delta rule actually works" gives the update, section "Kimi Delta
// Attention: the load-bearing choice" the per-channel gate and the blockwise
// organisation on matrix units; section "Training infrastructure:
// quantization-aware from SFT onward" that the layer is trained) is regrouped
// per 64-token chunk.  With G_r the inclusive cumulative log2-decay of each
// channel within the chunk (gam_r = 2^G_r, gam_L its value at the last token),
// entering state S0 and B = Diag(b):
//     Kt = K (.) gam,  Qt = Q (.) gam,  Ke = K (.) gam_L / gam   (row-wise, per channel)
//     A_ri = sum_c k_rc k_ic 2^(G_rc - G_ic)  (i < r),   P_ri = sum_c q_rc k_ic 2^(G_rc - G_ic)  (i <= r)
//     T = (I + B A)^-1,  X = Kt S0,  W = V - X,  U = T B W
//     O = Qt S0 + P U,   S1 = Diag(gam_L) S0 + Ke^T U.
// Given dO and the gradient dS1 in the leaving state, the chain rule gives
//     dU = P^T dO + Ke dS1,   dW' = T^T dU  (the gradient in B W),  dV = B dW'
//     dS0 = Diag(gam_L) dS1 + Qt^T dO - Kt^T B dW'
//     dQt = dO S0^T,  dKt = -B dW' S0^T,  dKe = U dS1^T,  dgam_L = rowsum(dS1 (.) S0)
//     dP = dO U^T (i <= r),  dT = dU (B W)^T,  dM = -T^T dT T^T,  dA = B dM (i < r)
//     db_r = sum_j dW'_rj W_rj + sum_i dM_ri A_ri
// and, through the decay factors, for every channel c (natural-log units:
// 2^(G_r - G_i) = e^(L_r - L_i) with L the cumulative log-decay)
//     dq_r += sum_{i<=r} dP_ri k_i e^(L_r - L_i),   dk_r += sum_{i<r} dA_ri k_i e^(L_r - L_i)
//     dk_i += sum_{r>=i} (dP_ri q_r + dA_ri k_r) e^(L_r - L_i)
// The gate's gradient comes from shifting L_r = sum_{j' <= r} log a_j' by the
// same amount for every r >= j (that is, changing log a_j): Qt_r and Kt_r
// (r >= j), Ke_r (r < j) and gam_L scale with it, and so do A_ri and P_ri
// for r >= j > i, so
//     d log a_j = sum_{r >= j} (Qt dQt + Kt dKt)_r + sum_{r < j} (Ke dKe)_r
//               + gam_L dgam_L + sum_{r >= j > i} X_ri,
//     X_ri = (dA_ri k_r + dP_ri q_r) k_i e^(L_r - L_i).
// Every term carries the decay over token j, so where that decay (or the
// state entering token j) vanishes, the gradient comes out as small as it
// is; the equivalent reverse sum over r >= j of the per-row derivatives would
// leave the rounding residue of terms that cancel.
//
// Kernels (one head of one sequence is a "unit"; chunks are numbered per head
// by the id floor(row0 / 64) + sequence + chunk, unique and below rows / 64 +
// sequences + 1, so dense and packed input share one workspace layout):
//   prep   (one workgroup per chunk)  A, P and T of every chunk;
//   states (one per unit, in order)   the entering state S0 of every chunk, and
//                                     W, parked in dk;
//   dstate (one per unit, reversed)   the gradient dS1 in every chunk's leaving
//                                     state, dU (parked in d log a), and the
//                                     initial-state gradient;
//   grads  (one per chunk)            first the gradient part: dV, the S0/dS1
//                                     parts of dq, dk and dL, db's first term,
//                                     dP and dT; then the intra-chunk part: dM,
//                                     dA, db's second term, the decay products
//                                     and their cross sums, the A/P part of
//                                     d log a, and the totals.
// The parked intermediates use the gradient buffers as scratch: each chunk's
// rows of its own head, written by a sweep and read back by the grads kernel
// of the same chunk before it writes the gradients there.
//
// Memory instructions follow a few rules that the timings showed to matter on
// this hardware: all global loads of a phase are issued before its first
// store and before the first use of any of them (loads and stores retire in
// order, so a wait for a load also waits for every earlier store); no load
// sits under a condition and no loaded value is converted or selected right
// after its load (either makes the compiler wait for the data on the spot);
// and a wave keeps at most 63 memory instructions in flight, so stores that
// would follow a chunk's requests are issued before them.
//
// Matrix products run on v_mfma_f32_16x16x32_bf16 with every operand split
// into hi + lo bf16 (hi*hi + hi*lo + lo*hi, fp32 accumulation), as in the
// prefill.  Operands in LDS are stored as "images": 16 x 32 tiles in lane
// order, so a fragment is one conflict-free 16-byte read per lane.  State-sized
// matrices stay in accumulator layout in registers; with the contraction index
// of a 32-step bound to (lane group g, slot j) as 16 (j >> 2) + 4 g + (j & 3),
// two accumulator tiles are directly the B operand of the next product (PERM
// images use the same binding for their A operand).
//
// Decay factors never overflow: in the off-diagonal 16 x 16 blocks (rows r in
// block R, columns i in an earlier block) 2^(G_r - G_i) is split at the last
// token of block R - 1 into two factors <= 1.  Inside the diagonal blocks it
// is split at the block's 8th token where both factors stay within 2^96, and
// formed pairwise on the vector ALUs for the other channels.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <type_traits>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int CH = 64;                      // tokens per chunk
constexpr int SS = kDim * kDim;             // floats per state
constexpr int TSZ = CH * CH;                // floats per 64 x 64 tile
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct ChunkBwdArgs {
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    const bf16_t* beta;
    const float* la;
    const float* d_o;
    const int32_t* cu;   // packed row offsets [n_seq + 1], or null (dense: T rows each)
    int64_t T;
    int64_t n_seq;
    int H;
    const float* s0;     // [n_seq, H, 128, 128] or null (zeros)
    const float* d_sT;   // [n_seq, H, 128, 128] or null (zeros)
    float* dq;
    float* dk;
    float* dv;
    float* dbeta;
    float* dla;
    float* ds0;          // [n_seq, H, 128, 128] or null (not written)
    float* ws_s0;        // [ids][H][128][128]  entering state of every chunk
    float* ws_ds;        // [ids][H][128][128]  gradient in every chunk's leaving state
    float* ws_apt;       // [ids][H][3][64][64] A, P, T
};

__device__ __forceinline__ int64_t seq_row0(const ChunkBwdArgs& a, int64_t n)
{
    return a.cu ? static_cast<int64_t>(a.cu[n]) : n * a.T;
}
__device__ __forceinline__ int64_t seq_len(const ChunkBwdArgs& a, int64_t n)
{
    return a.cu ? static_cast<int64_t>(a.cu[n + 1]) - a.cu[n] : a.T;
}
__device__ __forceinline__ int64_t chunk_id(int64_t row0, int64_t n, int64_t c)
{
    return (row0 >> 6) + n + c;
}

// Chunk id -> (sequence, chunk); false for ids that name no chunk.
__device__ bool locate(const ChunkBwdArgs& a, int64_t id, int64_t& n, int64_t& c)
{
    int64_t lo = 0, hi = a.n_seq;  // the last n with chunk_id(row0(n), n, 0) <= id
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (chunk_id(seq_row0(a, mid), mid, 0) <= id) lo = mid;
        else hi = mid;
    }
    n = lo;
    c = id - chunk_id(seq_row0(a, lo), lo, 0);
    return c >= 0 && c * CH < seq_len(a, lo);
}

// Workgroup barrier for LDS only: each wave's LDS reads and writes complete
// before it, while its global loads and stores stay in flight (a
// __syncthreads() would wait for those too).  The memory clobber keeps the
// compiler from moving memory accesses across it.  No kernel of this file
// reads, within one launch, global memory that another wave wrote.
__device__ __forceinline__ void lds_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Element i of an array at a wave-uniform base, addressed by a 32-bit byte
// offset (the base stays in scalar registers; i * sizeof(T) < 2^32).
template <typename T>
__device__ __forceinline__ T& at(T* base, uint32_t i)
{
    using C = typename std::conditional<std::is_const<T>::value, const char, char>::type;
    return *reinterpret_cast<T*>(reinterpret_cast<C*>(base) + i * static_cast<uint32_t>(sizeof(T)));
}

// A 128 x 128 fp32 state in accumulator layout: element (16 tt + 4 g + x,
// col) in X[tt][x], lane offset 4 g * 128 + col; the row's part of the
// address stays in the (scalar) base.
__device__ __forceinline__ void state_load(const float* src, uint32_t lo, f32x4 (&X)[8])
{
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int x = 0; x < 4; ++x) X[tt][x] = src ? at(src + (16 * tt + x) * kDim, lo) : 0.f;
}
__device__ __forceinline__ void state_store(float* dst, uint32_t lo, const f32x4 (&X)[8])
{
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int x = 0; x < 4; ++x) at(dst + (16 * tt + x) * kDim, lo) = X[tt][x];
}

// Chunk intermediates parked by the state sweeps in a [rows][H][128] fp32
// buffer, for lane (column col, lane group g) and row block m, rows
// 16 m + 4 g + x.  In a full chunk the four values of one column go to one
// 16-byte slot: rows 4q .. 4q + 3 (q = 4 m + g) of column c are kept at row
// 4q + c / 32, columns 4 (c mod 32) .. + 3 (a permutation inside the four
// rows, so one vector store or load per group instead of four).  A partial
// chunk keeps every row r < L at its own place.  `base` points at the
// chunk's first row for this head; rs is the row stride in floats.
__device__ __forceinline__ void park4(float* base, uint32_t rs, int m, int g, int col, int L, f32x4 v)
{
    if (L == CH) {
        const uint32_t lo = (4 * g + (col >> 5)) * rs + 4 * (col & 31);
        at(reinterpret_cast<f32x4*>(base + 16 * m * rs), lo >> 2) = v;
    } else {
#pragma unroll
        for (int x = 0; x < 4; ++x)
            if (16 * m + 4 * g + x < L) at(base + (16 * m + x) * rs, 4 * g * rs + col) = v[x];
    }
}
// All four row blocks of a lane (one branch for the four).
__device__ __forceinline__ void park_all(float* base, uint32_t rs, int g, int col, int L, const f32x4 (&v)[4])
{
    if (L == CH) {
        const uint32_t lo = ((4 * g + (col >> 5)) * rs + 4 * (col & 31)) >> 2;
#pragma unroll
        for (int m = 0; m < 4; ++m) at(reinterpret_cast<f32x4*>(base + 16 * m * rs), lo) = v[m];
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int x = 0; x < 4; ++x)
                if (16 * m + 4 * g + x < L) at(base + (16 * m + x) * rs, 4 * g * rs + col) = v[m][x];
    }
}
// The parked group back (rows from L on read row 0: to be replaced where used).
__device__ __forceinline__ f32x4 unpark4(const float* base, uint32_t rs, int m, int g, int col, int L)
{
    if (L == CH) {
        const uint32_t lo = (4 * g + (col >> 5)) * rs + 4 * (col & 31);
        return at(reinterpret_cast<const f32x4*>(base + 16 * m * rs), lo >> 2);
    }
    f32x4 v;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int r = 16 * m + 4 * g + x;
        v[x] = at(base, (r < L ? r : 0) * rs + col);
    }
    return v;
}

// The wave's index in the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// x from another lane of the same row of 16, by a DPP control (a vector-ALU
// operand modifier, no LDS traffic): quad_perm [1,0,3,2] swaps neighbours,
// [2,3,0,1] pairs, row_half_mirror reverses each group of 8, row_ror:n
// rotates the row by n.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppSwap1 = 0xB1, kDppSwap2 = 0x4E, kDppHalfMirror = 0x141;
template <int N>
__device__ __forceinline__ float row_ror(float x) { return dpp_mov<0x120 + N>(x); }

// the sum over the 16 lanes of a row, in each of them
__device__ __forceinline__ float row_sum16(float x)
{
    x += row_ror<8>(x);
    x += row_ror<4>(x);
    x += row_ror<2>(x);
    return x + row_ror<1>(x);
}
// the sum over each aligned group of 8 lanes, in each of them
__device__ __forceinline__ float group_sum8(float x)
{
    x += dpp_mov<kDppSwap1>(x);
    x += dpp_mov<kDppSwap2>(x);
    return x + dpp_mov<kDppHalfMirror>(x);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// ---------------------------------------------------------------- splits

// x0, x1 -> (hi pair, lo pair) of bf16, each packed in 32 bits:
// hi = bf16(x) (nearest even), lo = bf16(x - hi).
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& h, uint32_t& l)
{
    h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
    uint32_t u = h;
    asm("" : "+v"(u));  // read the hi values back from the packed bits
    l = __builtin_bit_cast(uint32_t,
                           __builtin_convertvector((f32x2){x0 - bf_lo(u), x1 - bf_hi(u)}, bf16x2));
}

// Eight values -> hi and lo bf16x8.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& h, bf16x8& l)
{
    uint32_t hu[4], lu[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) split2(x[2 * j], x[2 * j + 1], hu[j], lu[j]);
    h = __builtin_bit_cast(bf16x8, (uint4){hu[0], hu[1], hu[2], hu[3]});
    l = __builtin_bit_cast(bf16x8, (uint4){lu[0], lu[1], lu[2], lu[3]});
}

// Two accumulator tiles (rows 4g..4g+3 of tiles t0 and t1 in lane group g) as
// the B operand of a product summing over their rows (PERM binding).
__device__ __forceinline__ void bfrag(f32x4 t0, f32x4 t1, bf16x8& h, bf16x8& l)
{
    const float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
    split8(x, h, l);
}

// hi*hi + hi*lo + lo*hi
__device__ __forceinline__ f32x4 mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
    return c;
}

// ---------------------------------------------------------------- images
//
// An image of an R x K matrix Z (R a multiple of 16, K of 32) holds its 16 x 32
// tiles (row block rb, k-step s: tile rb * (K / 32) + s) in lane order: lane
// l = (row & 15) + 16 g keeps the 8 slots j of its row for slot group g, slot
// (g, j) holding k index 32 s + 8 g + j (natural) or 32 s + 16 (j >> 2) + 4 g +
// (j & 3) (PERM).  The hi plane comes first, the lo plane `plane` bytes later
// (plane = R * K * 2).

template <bool PERM>
__device__ __forceinline__ int img_off(int row, int kidx, int ks)
{
    const int kk = kidx & 31;
    int g, j;
    if (PERM) {
        g = (kk >> 2) & 3;
        j = ((kk >> 4) << 2) | (kk & 3);
    } else {
        g = kk >> 3;
        j = kk & 7;
    }
    return (((row >> 4) * ks + (kidx >> 5)) << 10) + (((row & 15) + 16 * g) << 4) + (j << 1);
}

// Store the split pair (x0 at kidx, x1 at kidx + 1; kidx even).
template <bool PERM>
__device__ __forceinline__ void img_put2(char* img, int plane, int row, int kidx, int ks, float x0,
                                         float x1)
{
    uint32_t h, l;
    split2(x0, x1, h, l);
    const int off = img_off<PERM>(row, kidx, ks);
    *reinterpret_cast<uint32_t*>(img + off) = h;
    *reinterpret_cast<uint32_t*>(img + plane + off) = l;
}

__device__ __forceinline__ void img_frag(const char* img, int plane, int tile, int lane, bf16x8& h,
                                         bf16x8& l)
{
    h = *reinterpret_cast<const bf16x8*>(img + (tile << 10) + (lane << 4));
    l = *reinterpret_cast<const bf16x8*>(img + plane + (tile << 10) + (lane << 4));
}

// ---------------------------------------------------------------- staging
//
// Thread t stages channels 2 (t & 63), +1 for tokens TOK * (t >> 6) .. +TOK-1
// of one chunk (NT / 64 token groups): log alpha becomes the inclusive
// cumulative log2-decay G (the group prefix through `tot`, an LDS array of
// NT / 64 x 128 floats), k and (WITHQ) q are widened.  Rows from L on are
// zeros (so they decay nothing and write nothing).
template <int NT>
struct Staged {
    static constexpr int TG = NT / 64;
    static constexpr int TOK = CH / TG;
    int c0;                 // first of the thread's two channels
    int r0;                 // first of its tokens
    float g[TOK][2];        // G
    float kk[TOK][2];
    float qq[TOK][2];
    float gl[2];            // G at the chunk's last token
};

// The raw inputs a thread stages for one chunk, requested ahead of their use.
template <int NT, bool WITHQ>
struct ChunkRaw {
    static constexpr int TOK = Staged<NT>::TOK;
    float2 la[TOK];
    uint32_t k[TOK];
    uint32_t q[WITHQ ? TOK : 1];
    int L;                  // the chunk's rows; the rest are zeroed by stage_raw
};

template <int NT, bool WITHQ>
__device__ __forceinline__ void request(const ChunkBwdArgs& a, int64_t row0c, int L, int h,
                                        ChunkRaw<NT, WITHQ>& p)
{
    constexpr int TOK = Staged<NT>::TOK;
    const int t = threadIdx.x;
    const int c0 = 2 * (t & 63), r0 = TOK * wave_id();
    // wave-uniform bases and 32-bit lane offsets
    const int64_t base = (row0c * a.H + h) * kDim;
    const float* la = a.la + base;
    const bf16_t* k = a.k + base;
    const bf16_t* q = a.q + base;
    const uint32_t rstride = static_cast<uint32_t>(a.H) * kDim;
    // Rows past the chunk's end load row 0 (always present) and are zeroed
    // at staging, not here: a load under a condition is compiled as a branch
    // that waits for it, and so is a select right after the load.
    p.L = L;
#pragma unroll
    for (int j = 0; j < TOK; ++j) {
        const int r = r0 + j;
        const uint32_t e = static_cast<uint32_t>(c0) + static_cast<uint32_t>(r < L ? r : 0) * rstride;
        p.la[j] = at(reinterpret_cast<const float2*>(la), e >> 1);
        p.k[j] = at(reinterpret_cast<const uint32_t*>(k), e >> 1);
        if (WITHQ) p.q[j] = at(reinterpret_cast<const uint32_t*>(q), e >> 1);
    }
}

// The cumulative log2-decay of the requested inputs (one barrier, for the
// group prefix through `tot`); rows from L on are zeroed in p first.
template <int NT, bool WITHQ>
__device__ __forceinline__ void stage_raw(ChunkRaw<NT, WITHQ>& p, float* tot, Staged<NT>& s)
{
    constexpr int TG = Staged<NT>::TG, TOK = Staged<NT>::TOK;
    const int t = threadIdx.x;
    s.c0 = 2 * (t & 63);
    s.r0 = TOK * wave_id();
#pragma unroll
    for (int j = 0; j < TOK; ++j) {
        const bool in = s.r0 + j < p.L;
        p.la[j] = in ? p.la[j] : make_float2(0.f, 0.f);
        p.k[j] = in ? p.k[j] : 0u;
        if (WITHQ) p.q[j] = in ? p.q[j] : 0u;
    }
    float run0 = 0.f, run1 = 0.f;
#pragma unroll
    for (int j = 0; j < TOK; ++j) {
        run0 += p.la[j].x * kLog2e;
        run1 += p.la[j].y * kLog2e;
        s.g[j][0] = run0;
        s.g[j][1] = run1;
        s.kk[j][0] = bf_lo(p.k[j]);
        s.kk[j][1] = bf_hi(p.k[j]);
        s.qq[j][0] = WITHQ ? bf_lo(p.q[j]) : 0.f;
        s.qq[j][1] = WITHQ ? bf_hi(p.q[j]) : 0.f;
    }
    tot[wave_id() * kDim + s.c0] = run0;
    tot[wave_id() * kDim + s.c0 + 1] = run1;
    lds_sync();
    float p0 = 0.f, p1 = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int u = 0; u < TG; ++u) {
        const float x0 = tot[u * kDim + s.c0], x1 = tot[u * kDim + s.c0 + 1];
        if (u < wave_id()) {
            p0 += x0;
            p1 += x1;
        }
        a0 += x0;
        a1 += x1;
    }
#pragma unroll
    for (int j = 0; j < TOK; ++j) {
        s.g[j][0] += p0;
        s.g[j][1] += p1;
    }
    s.gl[0] = a0;
    s.gl[1] = a1;
}

// beta of the chunk's row t mod 64 as raw bits, loaded without a branch (a
// row from L on reads row 0: its value is to be replaced by zero where it is
// used), to be widened where it is staged
__device__ __forceinline__ bf16_t beta_raw(const ChunkBwdArgs& a, int64_t row0c, int L, int h)
{
    const int t = threadIdx.x & (CH - 1);
    return a.beta[(row0c + (t < L ? t : 0)) * a.H + h];
}

// log alpha, k and q of one chunk, four channels per thread: thread t takes
// channels 4 (t mod 32) .. +3 of the TOK tokens TOK (t / 32) .. +TOK-1, so
// that each token is one 16-byte load of log alpha and one 8-byte load each
// of k and q.  Rows from L on load row 0 and are zeroed when staged.
template <int NT>
struct Raw4 {
    static constexpr int TOK = 32 * CH / NT;
    float4 la[TOK];
    uint2 k[TOK], q[TOK];
    int L;
};

template <int NT>
__device__ __forceinline__ void request4(const ChunkBwdArgs& a, int64_t row0c, int L, int h, Raw4<NT>& p)
{
    constexpr int TOK = Raw4<NT>::TOK;
    const int t = threadIdx.x;
    const int c0 = 4 * (t & 31), r0 = TOK * (t >> 5);
    const int64_t base = (row0c * a.H + h) * kDim;
    const uint32_t rstride = static_cast<uint32_t>(a.H) * kDim;
    p.L = L;
#pragma unroll
    for (int j = 0; j < TOK; ++j) {
        const int r = r0 + j;
        const uint32_t e4 = (static_cast<uint32_t>(c0) + static_cast<uint32_t>(r < L ? r : 0) * rstride) >> 2;
        p.la[j] = at(reinterpret_cast<const float4*>(a.la + base), e4);
        p.k[j] = at(reinterpret_cast<const uint2*>(a.k + base), e4);
        p.q[j] = at(reinterpret_cast<const uint2*>(a.q + base), e4);
    }
}

// The cumulative log2-decay G of the thread's elements (rows from L on zeroed
// in p first: they decay nothing) and G at the chunk's last token; one
// barrier, for the prefix over the waves through tot (NT / 64 x 128 floats).
// The two halves of a wave hold neighbouring token groups.
template <int NT>
__device__ __forceinline__ void stage4(Raw4<NT>& p, float* tot, float4 (&gv)[Raw4<NT>::TOK], float4& gl)
{
    constexpr int TOK = Raw4<NT>::TOK;
    const int t = threadIdx.x, c0 = 4 * (t & 31), r0 = TOK * (t >> 5);
    float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < TOK; ++j) {
        const bool in = r0 + j < p.L;
        const float4 x = p.la[j];
        p.k[j] = in ? p.k[j] : make_uint2(0u, 0u);
        p.q[j] = in ? p.q[j] : make_uint2(0u, 0u);
        run.x += in ? x.x * kLog2e : 0.f;
        run.y += in ? x.y * kLog2e : 0.f;
        run.z += in ? x.z * kLog2e : 0.f;
        run.w += in ? x.w * kLog2e : 0.f;
        gv[j] = run;
    }
    const float4 other = make_float4(__shfl_xor(run.x, 32), __shfl_xor(run.y, 32), __shfl_xor(run.z, 32),
                                     __shfl_xor(run.w, 32));
    const int w = wave_id();
    const bool upper = (t & 32) != 0;
    if (!upper)
        *reinterpret_cast<float4*>(&tot[w * kDim + c0]) =
            make_float4(run.x + other.x, run.y + other.y, run.z + other.z, run.w + other.w);
    lds_sync();
    float4 pre = upper ? other : make_float4(0.f, 0.f, 0.f, 0.f), all = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < NT / 64; ++u) {
        const float4 x = *reinterpret_cast<const float4*>(&tot[u * kDim + c0]);
        if (u < w) pre = make_float4(pre.x + x.x, pre.y + x.y, pre.z + x.z, pre.w + x.w);
        all = make_float4(all.x + x.x, all.y + x.y, all.z + x.z, all.w + x.w);
    }
#pragma unroll
    for (int j = 0; j < TOK; ++j)
        gv[j] = make_float4(gv[j].x + pre.x, gv[j].y + pre.y, gv[j].z + pre.z, gv[j].w + pre.w);
    gl = all;
}

// A 64 x 64 fp32 tile from global memory into an image: TRANS = false stores
// Z[r][i] at (row r, k i), TRANS = true at (row i, k r); PERM binding.  The
// loads (request_tile) come apart from the stores (tile_put) so that they can
// be issued a chunk ahead.  Each thread loads two 16-byte pieces: rows r and
// r + 32 (TRANS = false) or the rows 2p, 2p + 1 of one row pair p (TRANS =
// true), columns 4 (t mod 16) .. +3.
template <int NT>
struct TileRaw {
    static_assert(NT == 512, "two 16-byte pieces per thread");
    float4 x[2];
};

template <bool TRANS, int NT>
__device__ __forceinline__ void request_tile(const float* src, TileRaw<NT>& p)
{
    uint32_t tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // offsets recomputed per call, not kept across a loop
    const uint32_t i = 4 * (tid & 15);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t r = TRANS ? 2 * (tid >> 4) + j : (tid >> 4) + 32 * j;
        p.x[j] = at(reinterpret_cast<const float4*>(src), (r * CH + i) >> 2);
    }
}

template <bool TRANS, int NT>
__device__ __forceinline__ void tile_put(const TileRaw<NT>& p, char* img)
{
    constexpr int plane = CH * CH * 2;
    // (the addresses are recomputed at every call rather than kept in
    // registers across a caller's loop: the thread index is made opaque)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int i = 4 * (tid & 15);
    if (!TRANS) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = (tid >> 4) + 32 * j;
            img_put2<true>(img, plane, r, i, 2, p.x[j].x, p.x[j].y);
            img_put2<true>(img, plane, r, i + 2, 2, p.x[j].z, p.x[j].w);
        }
    } else {
        // the pair (Z[r][i + u], Z[r + 1][i + u]) is k = r, r + 1 of row i + u
        const int r = 2 * (tid >> 4);
        img_put2<true>(img, plane, i, r, 2, p.x[0].x, p.x[1].x);
        img_put2<true>(img, plane, i + 1, r, 2, p.x[0].y, p.x[1].y);
        img_put2<true>(img, plane, i + 2, r, 2, p.x[0].z, p.x[1].z);
        img_put2<true>(img, plane, i + 3, r, 2, p.x[0].w, p.x[1].w);
    }
}

// The 4 x 4 transpose of the float4 values of the four lanes of a quad: lane y
// holds row y (its four columns) and ends with column y (four rows), by two
// exchanges on DPP quad permutations.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 a)
{
    const int y = threadIdx.x & 3;
    const bool e = (y & 1) == 0, f = (y & 2) == 0;
    // lanes y and y ^ 1 swap the off-diagonal entries of their 2 x 2 blocks
    float r0 = dpp_mov<kDppSwap1>(e ? a[1] : a[0]);
    float r1 = dpp_mov<kDppSwap1>(e ? a[3] : a[2]);
    const f32x4 b = e ? (f32x4){a[0], r0, a[2], r1} : (f32x4){r0, a[1], r1, a[3]};
    // lanes y and y ^ 2 swap the off-diagonal 2 x 2 blocks
    r0 = dpp_mov<kDppSwap2>(f ? b[2] : b[0]);
    r1 = dpp_mov<kDppSwap2>(f ? b[3] : b[1]);
    return f ? (f32x4){b[0], b[1], r0, r1} : (f32x4){r0, r1, b[2], b[3]};
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// hi*hi + hi*lo + lo*hi on the 16x16x16 bf16 instruction
__device__ __forceinline__ f32x4 mma16(i16x4 ah, i16x4 al, i16x4 bh, i16x4 bl, f32x4 c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ void split4(float x0, float x1, float x2, float x3, i16x4& h, i16x4& l)
{
    uint32_t h0, l0, h1, l1;
    split2(x0, x1, h0, l0);
    split2(x2, x3, h1, l1);
    h = __builtin_bit_cast(i16x4, (uint2){h0, h1});
    l = __builtin_bit_cast(i16x4, (uint2){l0, l1});
}

// ================================================================ prep
//
// A, P and T of one chunk of one head (grid: chunk ids x heads; 256 threads,
// two workgroups per CU).  The ten lower 16 x 16 blocks of A and P run on the
// matrix cores (2.5 per wave), with 2^(G_r - G_i) split at a reference rho:
// the last token of block R - 1 for the six off-diagonal blocks (both factors
// <= 1), the block's 8th token for the four diagonal ones, where a channel is
// taken this way only if both factors stay within 2^96; the other ("unsafe")
// channels of a diagonal block are added pairwise on the vector ALUs.  Then
// T = (I + B A)^-1: its diagonal blocks by forward substitution (one wave per
// block, lane = (column, row quarter), quad sums over the lanes of a column),
// its off-diagonal blocks as T_RI = -T_RR sum_{I <= J < R} N_RJ T_JI in order
// of R - I (N = B A), on split-bf16 16x16x16 matrix instructions.  G, k and q
// live in LDS only until the A/P products are done; A, P and T then take their
// place.

constexpr int PREP_NT = 256;
constexpr int GLD = 132;     // fp32 row stride of the G tile
constexpr int BLD = 136;     // bf16 row stride of the k and q tiles
constexpr int TLD = 65;      // fp32 row stride of 64 x 64 tiles
constexpr int PLD = 68;      // fp32 row stride of the grads kernel's 64 x 64 tiles

// The six off-diagonal 16 x 16 blocks (row block, column block).
__device__ __forceinline__ void offdiag_block(int p, int& R, int& I)
{
    R = p < 1 ? 1 : p < 3 ? 2 : 3;
    I = p - (R * (R - 1)) / 2;
}

// x plus x from the lane that differs in lane bit 0 (XOR1) or bit 1 (XOR2).
template <int CTRL>
__device__ __forceinline__ float quad_add(float x)
{
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;

__global__ __launch_bounds__(PREP_NT, 2) void chunk_prep_kernel(const ChunkBwdArgs a)
{
    // phase 1: G | k | q;  phase 2 (the same bytes): A | P | T
    constexpr int OFF_G = 0, OFF_K = CH * GLD * 4, OFF_Q = OFF_K + CH * BLD * 2, P1 = OFF_Q + CH * BLD * 2;
    constexpr int OFF_A = 0, OFF_P = CH * TLD * 4, OFF_T = 2 * CH * TLD * 4, P2 = 3 * CH * TLD * 4;
    __shared__ __attribute__((aligned(16))) char sm[P1 > P2 ? P1 : P2];
    __shared__ float bs[CH];
    __shared__ float tot[(PREP_NT / 64) * kDim];
    __shared__ unsigned char unsafe_ch[4][kDim];   // per diagonal block and channel
    float* Gs = reinterpret_cast<float*>(sm + OFF_G);
    __bf16* Ks = reinterpret_cast<__bf16*>(sm + OFF_K);
    __bf16* Qs = reinterpret_cast<__bf16*>(sm + OFF_Q);
    float* As = reinterpret_cast<float*>(sm + OFF_A);
    float* Ps = reinterpret_cast<float*>(sm + OFF_P);
    float* Ts = reinterpret_cast<float*>(sm + OFF_T);

    const int H = a.H;
    const int64_t id = blockIdx.x / H;
    const int h = static_cast<int>(blockIdx.x - id * H);
    int64_t n, c;
    if (!locate(a, id, n, c)) return;
    const int64_t row0c = seq_row0(a, n) + c * CH;
    const int L = static_cast<int>(min<int64_t>(CH, seq_len(a, n) - c * CH));
    const int t = threadIdx.x, lane = t & 63, wave = wave_id(), g = lane >> 4, l16 = lane & 15;

    {
        Raw4<PREP_NT> raw;
        request4<PREP_NT>(a, row0c, L, h, raw);
        const bf16_t braw = beta_raw(a, row0c, L, h);   // in flight with the staging loads
        __builtin_amdgcn_sched_barrier(0);              // all requests issued before the first use
        float4 gv[Raw4<PREP_NT>::TOK], gl;
        stage4<PREP_NT>(raw, tot, gv, gl);
        if (t < CH) bs[t] = t < L ? widen(braw) : 0.f;
        const int c0 = 4 * (t & 31), r0 = Raw4<PREP_NT>::TOK * (t >> 5);
#pragma unroll
        for (int j = 0; j < Raw4<PREP_NT>::TOK; ++j) {
            const int r = r0 + j;
            *reinterpret_cast<float4*>(&Gs[r * GLD + c0]) = gv[j];
            *reinterpret_cast<uint2*>(&Ks[r * BLD + c0]) = raw.k[j];
            *reinterpret_cast<uint2*>(&Qs[r * BLD + c0]) = raw.q[j];
        }
    }
    lds_sync();
    if (t < kDim) {
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            const float g0 = Gs[(16 * R) * GLD + t], gm = Gs[(16 * R + 7) * GLD + t],
                        g1 = Gs[(16 * R + 15) * GLD + t];
            unsafe_ch[R][t] = (g0 - gm > 96.f || gm - g1 > 96.f) ? 1 : 0;
        }
    }
    lds_sync();

    // ---- A and P: block p = wave + 4 j; p < 4 the diagonal block p, else
    // the off-diagonal block p - 4.  Accumulators stay in registers until
    // every wave is done with G, k and q.
    f32x4 accA[3], accP[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        accA[j] = accP[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        const int p = wave + 4 * j;
        if (p >= 10) break;
        int R = p, I = p;
        if (p >= 4) offdiag_block(p - 4, R, I);
        const bool diag = R == I;
        const int rr = 16 * R + l16, ii = 16 * I + l16;
        const int rho_row = diag ? 16 * R + 7 : 16 * R - 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int cc = 32 * s + 8 * g;
            float fk[8], fq[8], fh[8];
            const bf16x8 kr = *reinterpret_cast<const bf16x8*>(&Ks[rr * BLD + cc]);
            const bf16x8 qr = *reinterpret_cast<const bf16x8*>(&Qs[rr * BLD + cc]);
            const bf16x8 ki = *reinterpret_cast<const bf16x8*>(&Ks[ii * BLD + cc]);
            const uint2 us = *reinterpret_cast<const uint2*>(&unsafe_ch[R][cc]);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const bool ok = !diag || (((jj < 4 ? us.x : us.y) >> (8 * (jj & 3))) & 0xffu) == 0;
                const float rho = Gs[rho_row * GLD + cc + jj];
                // (formed unconditionally, then selected: LDS reads under the
                // condition would become branches)
                const float fe = ex2(Gs[rr * GLD + cc + jj] - rho);
                const float he = (float)ki[jj] * ex2(rho - Gs[ii * GLD + cc + jj]);
                const float fr = ok ? fe : 0.f;
                fk[jj] = (float)kr[jj] * fr;
                fq[jj] = (float)qr[jj] * fr;
                fh[jj] = ok ? he : 0.f;
            }
            bf16x8 kh, kl, qh, ql, hh, hl;
            split8(fk, kh, kl);
            split8(fq, qh, ql);
            split8(fh, hh, hl);
            accA[j] = mma3(kh, kl, hh, hl, accA[j]);
            accP[j] = mma3(qh, ql, hh, hl, accP[j]);
        }
        if (diag) {
            // the unsafe channels of this diagonal block, pairwise (i <= r)
            const bool any = __any(unsafe_ch[R][lane] | unsafe_ch[R][lane + 64]);
            if (any) {
                for (int ch = 0; ch < kDim; ++ch) {
                    if (!unsafe_ch[R][ch]) continue;   // the same for every lane
                    const int i = 16 * R + l16;
                    const float gi = Gs[i * GLD + ch], ki = (float)Ks[i * BLD + ch];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int r = 16 * R + 4 * g + x;
                        if (i <= r) {
                            const float e = ki * ex2(Gs[r * GLD + ch] - gi);
                            accA[j][x] += (float)Ks[r * BLD + ch] * e;
                            accP[j][x] += (float)Qs[r * BLD + ch] * e;
                        }
                    }
                }
            }
        }
    }
    lds_sync();   // G, k and q are dead: A, P and T take their bytes
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int p = wave + 4 * j;
        if (p >= 10) break;
        int R = p, I = p;
        if (p >= 4) offdiag_block(p - 4, R, I);
        const int i = 16 * I + l16;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = 16 * R + 4 * g + x;
            As[r * TLD + i] = i < r ? accA[j][x] : 0.f;
            Ps[r * TLD + i] = i <= r ? accP[j][x] : 0.f;
        }
    }
    lds_sync();

    // ---- T = (I + N)^-1, N = B A (strictly lower).  Diagonal block R on wave
    // R: lane (jc, p) holds rows 4p..4p+3 of column jc of T_RR.
    {
        const int R = wave, jc = lane >> 2, pq = lane & 3;
        float4 nv[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int r = 16 * R + rr;
            const float br = bs[r];
            const float* ar = &As[r * TLD + 16 * R + 4 * pq];
            nv[rr] = make_float4(br * ar[0], br * ar[1], br * ar[2], br * ar[3]);
        }
        float tv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            // N is strictly lower and the rows of T not yet solved are zero
            float sum = nv[rr].x * tv[0] + nv[rr].y * tv[1] + nv[rr].z * tv[2] + nv[rr].w * tv[3];
            sum = quad_add<kQuadXor1>(sum);
            sum = quad_add<kQuadXor2>(sum);
            const float tr = (rr == jc ? 1.f : 0.f) - sum;
            if (pq == (rr >> 2)) tv[rr & 3] = tr;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) Ts[(16 * R + 4 * pq + m) * TLD + 16 * R + jc] = tv[m];
    }
    lds_sync();
    // Off-diagonal blocks by distance d = R - I (wave w < 4 - d takes R = d + w,
    // I = w), on split-bf16 16x16x16 matrix instructions:
    //   Y = B_R sum_{I <= J < R} A_RJ T_JI,   T_RI = -T_RR Y.
    // Y comes out in accumulator layout, which is the B operand of the second
    // product as it stands.
    for (int d = 1; d < 4; ++d) {
        if (wave < 4 - d) {
            const int R = d + wave, I = wave;
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 y = z;
            for (int J = I; J < R; ++J) {
                float av[4], bv[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    av[x] = As[(16 * R + l16) * TLD + 16 * J + 4 * g + x];
                    bv[x] = Ts[(16 * J + 4 * g + x) * TLD + 16 * I + l16];
                }
                i16x4 ah, al, bh, bl;
                split4(av[0], av[1], av[2], av[3], ah, al);
                split4(bv[0], bv[1], bv[2], bv[3], bh, bl);
                y = mma16(ah, al, bh, bl, y);
            }
            float by[4], tv[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                by[x] = bs[16 * R + 4 * g + x] * y[x];
                tv[x] = Ts[(16 * R + l16) * TLD + 16 * R + 4 * g + x];
            }
            i16x4 ah, al, bh, bl;
            split4(tv[0], tv[1], tv[2], tv[3], ah, al);
            split4(by[0], by[1], by[2], by[3], bh, bl);
            const f32x4 tr = mma16(ah, al, bh, bl, z);
#pragma unroll
            for (int x = 0; x < 4; ++x) Ts[(16 * R + 4 * g + x) * TLD + 16 * I + l16] = -tr[x];
        }
        lds_sync();
    }

    // ---- out: A (i < r), P (i <= r), T (i < r, unit diagonal), zeros elsewhere
    float* dst = a.ws_apt + (id * H + h) * (3 * TSZ);
    for (int e = 4 * t; e < TSZ; e += 4 * PREP_NT) {
        const int r = e >> 6, i0 = e & 63;
        float4 va, vp, vt;
        float* pa = &va.x;
        float* pp = &vp.x;
        float* pt = &vt.x;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u;
            // (read unconditionally, then selected: reads under the condition
            // would become branches)
            const float xa = As[r * TLD + i], xp = Ps[r * TLD + i], xt = Ts[r * TLD + i];
            pa[u] = i < r ? xa : 0.f;
            pp[u] = i <= r ? xp : 0.f;
            pt[u] = i < r ? xt : (i == r ? 1.f : 0.f);
        }
        *reinterpret_cast<float4*>(dst + e) = va;
        *reinterpret_cast<float4*>(dst + TSZ + e) = vp;
        *reinterpret_cast<float4*>(dst + 2 * TSZ + e) = vt;
    }
}

// ================================================================ states
//
// The entering state S0 of every chunk of one unit (grid: units; 512 threads).
// Wave w holds state columns 16w..16w+15 in accumulator layout: S[t][x] is
// row 16t + 4g + x of column 16w + (lane & 15), g = lane >> 4.
//   X = Kt S0,  W = V - X,  U = T B W,  S1 = Diag(gam_L) S0 + Ke^T U.

constexpr int SEQ_NT = 512;

__global__ __launch_bounds__(SEQ_NT, 1) void chunk_states_kernel(const ChunkBwdArgs a)
{
    constexpr int KT_PL = CH * kDim * 2, KE_PL = kDim * CH * 2, T_PL = CH * CH * 2;
    __shared__ __attribute__((aligned(16))) char KT[2 * KT_PL];   // Kt: rows r, k = channels
    __shared__ __attribute__((aligned(16))) char KE[2 * KE_PL];   // Ke^T: rows c, k = tokens
    __shared__ __attribute__((aligned(16))) char TI[2 * T_PL];    // T: rows r, k = i
    // V rows (bf16) at a row stride of VLD elements: the four lane groups of a
    // wave read rows 4 apart, which then fall in disjoint banks
    constexpr int VLD = kDim + 8;
    __shared__ __attribute__((aligned(16))) __bf16 VS[CH * VLD];
    __shared__ float tot[(SEQ_NT / 64) * kDim];
    __shared__ float bs[CH], gls[kDim];

    const int H = a.H;
    const int64_t n = blockIdx.x / H;
    const int h = static_cast<int>(blockIdx.x - n * H);
    const int64_t row0 = seq_row0(a, n), len = seq_len(a, n);
    const int64_t nch = (len + CH - 1) / CH;
    const int t = threadIdx.x, lane = t & 63, wave = wave_id(), g = lane >> 4;
    const int col = 16 * wave + (lane & 15);

    const uint32_t slo = 4 * g * kDim + col;
    f32x4 S[8];
    state_load(a.s0 ? a.s0 + (n * H + h) * SS : nullptr, slo, S);

    // The inputs of chunk c + 1 are requested while chunk c's products run:
    // log alpha and k, the T tile, V (row t / 8, columns 16 (t mod 8) .. +15)
    // and beta.
    ChunkRaw<SEQ_NT, false> raw;
    TileRaw<SEQ_NT> traw;
    uint4 vraw0, vraw1;   // (named registers: an array of two ended up in scratch memory)
    bf16_t braw = {0};   // raw bits, widened where staged (widening here would wait for the load)
    auto request_chunk = [&](int64_t c) {
        const int64_t row0c = row0 + c * CH;
        const int L = static_cast<int>(min<int64_t>(CH, len - c * CH));
        const int64_t id = chunk_id(row0, n, c);
        request_tile<false, SEQ_NT>(a.ws_apt + (id * H + h) * (3 * TSZ) + 2 * TSZ, traw);
        request<SEQ_NT, false>(a, row0c, L, h, raw);
        // rows from L on read row L - 1; they are replaced by zeros where the
        // values are consumed (a select here would wait for the loads)
        const bf16_t* vb = a.v + (row0c * H + h) * kDim;
        const uint32_t rs = H * kDim;
        const uint32_t ve = static_cast<uint32_t>(min(t >> 3, L - 1)) * rs + 16 * (t & 7);
        vraw0 = at(reinterpret_cast<const uint4*>(vb), ve >> 3);
        vraw1 = at(reinterpret_cast<const uint4*>(vb), (ve >> 3) + 1);
        braw = at(a.beta + row0c * H + h, static_cast<uint32_t>(min(t, L - 1)) * H);
    };
    if (nch > 0) request_chunk(0);

    // one chunk step; FULL: a chunk of 64 rows (every chunk but a sequence's
    // last), compiled apart so that its parking takes no branches
    auto step = [&](const int64_t c, auto full) {
        constexpr bool FULL = decltype(full)::value;
        const int64_t id = chunk_id(row0, n, c);
        const int64_t row0c = row0 + c * CH;
        const int L = FULL ? CH : static_cast<int>(min<int64_t>(CH, len - c * CH));
        lds_sync();  // the previous chunk's products are done with the images
        tile_put<false, SEQ_NT>(traw, TI);
        {
            uint4* vs = reinterpret_cast<uint4*>(&VS[(t >> 3) * VLD + 16 * (t & 7)]);
            vs[0] = vraw0;
            vs[1] = vraw1;
        }
        if (t < CH) bs[t] = t < L ? widen(braw) : 0.f;
        Staged<SEQ_NT> st;
        stage_raw<SEQ_NT, false>(raw, tot, st);
#pragma unroll
        for (int j = 0; j < Staged<SEQ_NT>::TOK; ++j) {
            const int r = st.r0 + j;
            img_put2<true>(KT, KT_PL, r, st.c0, 4, st.kk[j][0] * ex2(st.g[j][0]),
                           st.kk[j][1] * ex2(st.g[j][1]));
        }
#pragma unroll
        for (int j = 0; j < Staged<SEQ_NT>::TOK; j += 2) {
            const int r = st.r0 + j;
#pragma unroll
            for (int u = 0; u < 2; ++u)
                img_put2<true>(KE, KE_PL, st.c0 + u, r, 2, st.kk[j][u] * ex2(st.gl[u] - st.g[j][u]),
                               st.kk[j + 1][u] * ex2(st.gl[u] - st.g[j + 1][u]));
        }
        if (st.r0 == 0) {
            gls[st.c0] = ex2(st.gl[0]);
            gls[st.c0 + 1] = ex2(st.gl[1]);
        }
        lds_sync();
        if (c + 1 < nch) request_chunk(c + 1);

        // X = Kt S0 (sum over channels: B from S, 4 steps).  The checkpoint of
        // S0 is stored alongside, two row tiles per step, after the requests:
        // the stores' issue overlaps the products, and waiting for the
        // requests (loads and stores complete in order) does not wait for them.
        float* s0dst = a.ws_s0 + (id * H + h) * SS;
        f32x4 X[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) X[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 bh, bl;
            bfrag(S[2 * s], S[2 * s + 1], bh, bl);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                bf16x8 ah, al;
                img_frag(KT, KT_PL, m * 4 + s, lane, ah, al);
                X[m] = mma3(ah, al, bh, bl, X[m]);
            }
#pragma unroll
            for (int tt = 2 * s; tt < 2 * s + 2; ++tt)
#pragma unroll
                for (int x = 0; x < 4; ++x) at(s0dst + (16 * tt + x) * kDim, slo) = S[tt][x];
        }
        // W = V - X (parked in dk for the grads kernel), then B W; rows from
        // L on hold row L - 1 of V and are taken as zeros
        {
            float* wdst = a.dk + (row0c * H + h) * kDim;
            const uint32_t rs = H * kDim;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 w;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int r = 16 * m + 4 * g + x;
                    const float v = (float)VS[r * VLD + col];
                    w[x] = (FULL || r < L ? v : 0.f) - X[m][x];
                    X[m][x] = bs[r] * w[x];
                }
                park4(wdst, rs, m, g, col, L, w);
            }
        }
        // U = T (B W) (sum over tokens: 2 steps)
        f32x4 U[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) U[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 wh, wl;
            bfrag(X[2 * s], X[2 * s + 1], wh, wl);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                bf16x8 ah, al;
                img_frag(TI, T_PL, m * 2 + s, lane, ah, al);
                U[m] = mma3(ah, al, wh, wl, U[m]);
            }
        }
        // S1 = Diag(gam_L) S0 + Ke^T U
        bf16x8 uh[2], ul[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) bfrag(U[2 * s], U[2 * s + 1], uh[s], ul[s]);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
#pragma unroll
            for (int x = 0; x < 4; ++x) S[tt][x] *= gls[16 * tt + 4 * g + x];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8 ah, al;
                img_frag(KE, KE_PL, tt * 2 + s, lane, ah, al);
                S[tt] = mma3(ah, al, uh[s], ul[s], S[tt]);
            }
        }
    };
    // the full chunks in a loop of their own; a partial last chunk after it
    const int64_t nfull = len / CH;
    for (int64_t c = 0; c < nfull; ++c) step(c, std::true_type{});
    if (nfull < nch) step(nfull, std::false_type{});
}

// ================================================================ dstate
//
// The gradient dS1 in the leaving state of every chunk of one unit, last
// chunk first (grid: units; 512 threads; the layout of the states kernel),
// and the initial-state gradient:
//   dU = P^T dO + Ke dS1,  dW' = T^T dU,  dS0 = Diag(gam_L) dS1 + Qt^T dO - Kt^T B dW'.

__global__ __launch_bounds__(SEQ_NT, 1) void chunk_dstate_kernel(const ChunkBwdArgs a)
{
    constexpr int KE_PL = CH * kDim * 2, TT_PL = kDim * CH * 2, T_PL = CH * CH * 2;
    __shared__ __attribute__((aligned(16))) char KE[2 * KE_PL];    // Ke: rows i, k = channels
    __shared__ __attribute__((aligned(16))) char QTT[2 * TT_PL];   // Qt^T: rows c, k = tokens
    __shared__ __attribute__((aligned(16))) char KTT[2 * TT_PL];   // Kt^T: rows c, k = tokens
    __shared__ __attribute__((aligned(16))) char PT[2 * T_PL];     // P^T: rows i, k = r
    __shared__ __attribute__((aligned(16))) char TT[2 * T_PL];     // T^T: rows i, k = r
    __shared__ float tot[(SEQ_NT / 64) * kDim];
    __shared__ float bs[CH], gls[kDim];

    const int H = a.H;
    const int64_t n = blockIdx.x / H;
    const int h = static_cast<int>(blockIdx.x - n * H);
    const int64_t row0 = seq_row0(a, n), len = seq_len(a, n);
    const int64_t nch = (len + CH - 1) / CH;
    const int t = threadIdx.x, lane = t & 63, wave = wave_id(), g = lane >> 4;
    const int col = 16 * wave + (lane & 15);

    const uint32_t slo = 4 * g * kDim + col;
    f32x4 dS[8];
    state_load(a.d_sT ? a.d_sT + (n * H + h) * SS : nullptr, slo, dS);

    // The inputs of chunk c - 1 are requested while chunk c's products run:
    // log alpha, k and q, the P and T tiles, this thread's dO rows and beta.
    ChunkRaw<SEQ_NT, true> raw;
    TileRaw<SEQ_NT> praw, traw;
    f32x4 oraw[4];
    bf16_t braw = {0};   // raw bits, widened where staged (widening here would wait for the load)
    auto request_chunk = [&](int64_t c) {
        const int64_t row0c = row0 + c * CH;
        const int L = static_cast<int>(min<int64_t>(CH, len - c * CH));
        const float* apt = a.ws_apt + (chunk_id(row0, n, c) * H + h) * (3 * TSZ);
        request_tile<true, SEQ_NT>(apt + TSZ, praw);
        request_tile<true, SEQ_NT>(apt + 2 * TSZ, traw);
        request<SEQ_NT, true>(a, row0c, L, h, raw);
        // rows from L on read row L - 1; they are replaced by zeros where the
        // values are consumed (a select here would wait for the loads).  Lane
        // (g, 4 q + y) loads row 16 m + 4 g + y, columns 16 w + 4 q .. +3; a
        // quad transpose at staging gives it column 16 w + 4 q + y of the
        // four rows 16 m + 4 g + x.
        const float* ob = a.d_o + (row0c * H + h) * kDim;
        const uint32_t rs = H * kDim;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * m + 4 * g + (lane & 3);
            oraw[m] = at(reinterpret_cast<const f32x4*>(ob),
                         (16 * wave + 4 * ((lane & 15) >> 2) + static_cast<uint32_t>(min(r, L - 1)) * rs) >> 2);
        }
        braw = at(a.beta + row0c * H + h, static_cast<uint32_t>(min(t, L - 1)) * H);
    };
    if (nch > 0) request_chunk(nch - 1);

    // one chunk step; FULL: a chunk of 64 rows (every chunk but a sequence's
    // last), compiled apart so that its parking takes no branches
    auto step = [&](const int64_t c, auto full) {
        constexpr bool FULL = decltype(full)::value;
        const int64_t id = chunk_id(row0, n, c);
        const int64_t row0c = row0 + c * CH;
        const int L = FULL ? CH : static_cast<int>(min<int64_t>(CH, len - c * CH));
        lds_sync();
        tile_put<true, SEQ_NT>(praw, PT);
        tile_put<true, SEQ_NT>(traw, TT);
        if (t < CH) bs[t] = t < L ? widen(braw) : 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            oraw[m] = quad_transpose(oraw[m]);
#pragma unroll
            for (int x = 0; x < 4; ++x)
                if (16 * m + 4 * g + x >= L) oraw[m][x] = 0.f;
        }
        // dO in accumulator layout (rows r = 16m + 4g + x of column col), split
        bf16x8 oh[2], ol[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) bfrag(oraw[2 * s], oraw[2 * s + 1], oh[s], ol[s]);
        Staged<SEQ_NT> st;
        stage_raw<SEQ_NT, true>(raw, tot, st);
        // (the image addresses are recomputed every chunk rather than kept in
        // registers across the loop: the channel index is made opaque here)
        asm volatile("" : "+v"(st.c0));
#pragma unroll
        for (int j = 0; j < Staged<SEQ_NT>::TOK; ++j) {
            const int r = st.r0 + j;
            img_put2<true>(KE, KE_PL, r, st.c0, 4, st.kk[j][0] * ex2(st.gl[0] - st.g[j][0]),
                           st.kk[j][1] * ex2(st.gl[1] - st.g[j][1]));
        }
#pragma unroll
        for (int j = 0; j < Staged<SEQ_NT>::TOK; j += 2) {
            const int r = st.r0 + j;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float e0 = ex2(st.g[j][u]), e1 = ex2(st.g[j + 1][u]);
                img_put2<true>(QTT, TT_PL, st.c0 + u, r, 2, st.qq[j][u] * e0, st.qq[j + 1][u] * e1);
                img_put2<true>(KTT, TT_PL, st.c0 + u, r, 2, st.kk[j][u] * e0, st.kk[j + 1][u] * e1);
            }
        }
        if (st.r0 == 0) {
            gls[st.c0] = ex2(st.gl[0]);
            gls[st.c0 + 1] = ex2(st.gl[1]);
        }
        // the gradient in this chunk's leaving state, stored before the next
        // chunk's requests: a wave keeps at most 63 memory instructions in
        // flight, and these stores issued after the requests would have to
        // wait for the requests' data to make room
        state_store(a.ws_ds + (id * H + h) * SS, slo, dS);
        lds_sync();
        if (c > 0) request_chunk(c - 1);
        __builtin_amdgcn_sched_barrier(0);  // the requests go out before the products

        // dU = P^T dO + Ke dS1
        f32x4 dU[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            dU[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8 ah, al;
                img_frag(PT, T_PL, m * 2 + s, lane, ah, al);
                dU[m] = mma3(ah, al, oh[s], ol[s], dU[m]);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 sh, sl;
            bfrag(dS[2 * s], dS[2 * s + 1], sh, sl);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                bf16x8 ah, al;
                img_frag(KE, KE_PL, m * 4 + s, lane, ah, al);
                dU[m] = mma3(ah, al, sh, sl, dU[m]);
            }
            __builtin_amdgcn_sched_barrier(0);  // bounds the fragments in flight
        }
        // dW' = T^T dU, then -B dW'
        f32x4 nW[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) nW[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 uh, ul;
            bfrag(dU[2 * s], dU[2 * s + 1], uh, ul);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                bf16x8 ah, al;
                img_frag(TT, T_PL, m * 2 + s, lane, ah, al);
                nW[m] = mma3(ah, al, uh, ul, nW[m]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // dU parked in d log alpha for the grads kernel, then -B dW'
        __builtin_amdgcn_sched_barrier(0);
        {
            const int64_t base = (row0c * H + h) * kDim;
            const uint32_t rs = H * kDim;
            park_all(a.dla + base, rs, g, col, L, dU);
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int x = 0; x < 4; ++x) nW[m][x] *= -bs[16 * m + 4 * g + x];
        }
        __builtin_amdgcn_sched_barrier(0);
        // dS0 = Diag(gam_L) dS1 + Qt^T dO - Kt^T B dW'
        bf16x8 wh[2], wl[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) bfrag(nW[2 * s], nW[2 * s + 1], wh[s], wl[s]);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
#pragma unroll
            for (int x = 0; x < 4; ++x) dS[tt][x] *= gls[16 * tt + 4 * g + x];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8 ah, al;
                img_frag(QTT, TT_PL, tt * 2 + s, lane, ah, al);
                dS[tt] = mma3(ah, al, oh[s], ol[s], dS[tt]);
                img_frag(KTT, TT_PL, tt * 2 + s, lane, ah, al);
                dS[tt] = mma3(ah, al, wh[s], wl[s], dS[tt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // a partial last chunk (the first in this order) before the loop over
    // the full ones
    const int64_t nfull = len / CH;
    if (nfull < nch) step(nfull, std::false_type{});
    for (int64_t c = nfull - 1; c >= 0; --c) step(c, std::true_type{});
    if (a.ds0) state_store(a.ds0 + (n * H + h) * SS, slo, dS);
}

// ================================================================ grads: gradient part
//
// Per chunk of one head (512 threads; the first part of the grads kernel).
// Phase A, wave w on value columns 16w..16w+15 (accumulator layout):
// W = V - Kt S0 (parked in dk by the states kernel), dU (parked in d log alpha
// by the dstate kernel), dO; U = T B W and dW' = T^T dU formed again from the
// T tile;
//   writes dv = B dW' and the row sums of dW' (.) W (db, first term).
// Phase B, wave w on channels 16w..16w+15 (sums over the value columns j,
// from LDS images of dO, -B dW' and U and the rows of S0 and dS1 read from
// the workspaces as B operands):
//   dQt = dO S0^T, dKt = -B dW' S0^T, dKe = U dS1^T, dgam_L = rowsum(dS1 (.) S0);
//   forms dq = dQt gam, dk = dKt gam + dKe gam_L / gam and the S0 part of
//   d log a, kept in registers for the intra-chunk part (which adds its
//   terms and writes the totals); dP = dO U^T (lower blocks) into LDS.
// Phase C: dT = dU (B W)^T (lower blocks) from images of dU and B W, into LDS.

constexpr int INTRA_NT = SEQ_NT;   // the intra-chunk part runs in the same workgroup

// The intra-chunk part's inputs: the A and T tiles, requested while the
// gradient part still runs, and from the gradient part's staging the raw
// keys, queries (rows from L on zeroed) and beta.  G stays in the gradient
// part's LDS tile.
struct IntraReq {
    static constexpr int NE = TSZ / INTRA_NT / 4;   // 16-byte pieces per thread and tile
    f32x4 ar[NE], tr[NE];
    bf16_t braw;
    ChunkRaw<INTRA_NT, true> raw;
};

__device__ __forceinline__ void intra_request(const ChunkBwdArgs& a, int64_t id, int h, int64_t row0c, int L,
                                              IntraReq& rq)
{
    const int t = threadIdx.x;
    const f32x4* apt = reinterpret_cast<const f32x4*>(a.ws_apt + (id * a.H + h) * (3 * TSZ));
#pragma unroll
    for (int j = 0; j < IntraReq::NE; ++j) {
        const int e = t + j * INTRA_NT;   // 16-byte piece: row e / 16, columns 4 (e mod 16) .. +3
        rq.ar[j] = apt[e];
        rq.tr[j] = apt[2 * TSZ / 4 + e];
    }
}

// The gradient part's terms of dq, dk and d log alpha, held in registers for
// the intra-chunk part: row 16 m + 4 g + x, channel 16 w + l16 (the same
// thread owns the same elements in both parts).
struct Partials {
    float q[4][4], k[4][4], l[4][4];
};

constexpr int GR_KT_PL = CH * kDim * 2;
// LDS of the gradient part (phase B: dO | -B dW' | U;  phase C: dU | B W, and
// dT where U was).  dP and dT stay in LDS for the intra-chunk part.
struct GradsLds {
    char img[6 * GR_KT_PL];
    float Gs[CH * GLD];
    float tot[(SEQ_NT / 64) * kDim];
    float bs[CH], gLs[kDim], dbr[SEQ_NT / 64][CH], dpd[SEQ_NT / 64][CH];
    float Pd[CH * PLD];   // dP (i <= r; the blocks above the diagonal are not written)
};
// dT (fp32, row stride PLD) at the end of the image of U
constexpr int GR_DT_OFF = 6 * GR_KT_PL - CH * PLD * 4;
static_assert(CH * PLD * 4 <= 2 * GR_KT_PL, "dT fits where the image of U was");

__device__ __forceinline__ void grads_part(const ChunkBwdArgs& a, char* sm, IntraReq& rq, Partials& pp)
{
    constexpr int KT_PL = GR_KT_PL;
    constexpr int OFF_I0 = 0, OFF_I1 = 2 * KT_PL, OFF_I2 = 4 * KT_PL;
    GradsLds& S_ = *reinterpret_cast<GradsLds*>(sm);
    char* img = S_.img;
    float* Gs = S_.Gs;
    float* tot = S_.tot;
    float* bs = S_.bs;
    float* gLs = S_.gLs;
    float (*dbr)[CH] = S_.dbr;
    float (*dpd)[CH] = S_.dpd;
    float* Pd = S_.Pd;
    float* Dt = reinterpret_cast<float*>(img + GR_DT_OFF);

    const int H = a.H;
    const int64_t id = blockIdx.x / H;
    const int h = static_cast<int>(blockIdx.x - id * H);
    int64_t n, c;
    if (!locate(a, id, n, c)) return;
    const int64_t row0c = seq_row0(a, n) + c * CH;
    const int L = static_cast<int>(min<int64_t>(CH, seq_len(a, n) - c * CH));
    const int t = threadIdx.x, lane = t & 63, wave = wave_id(), g = lane >> 4, l16 = lane & 15;
    const int col = 16 * wave + l16;
    const int64_t rs = static_cast<int64_t>(H) * kDim;      // elements per token row
    const int64_t wslot = id * H + h;

    // ---- every global load of the chunk is issued here, before the first
    // store: one round of latency, and no wait for a load also waits for
    // earlier stores (loads and stores share one counter).  W and dU were
    // parked in dk and d log alpha by the state sweeps; U = T (B W) and
    // dW' = T^T dU are formed again here from the T tile, on the same
    // products the sweeps used.
    ChunkRaw<SEQ_NT, true>& raw = rq.raw;   // kept: the intra-chunk part stages its k and q
    request<SEQ_NT, true>(a, row0c, L, h, raw);
    rq.braw = beta_raw(a, row0c, L, h);
    const bf16_t& braw = rq.braw;
    TileRaw<SEQ_NT> traw;   // T, rows 2p and 2p + 1: both images from one load
    request_tile<true, SEQ_NT>(a.ws_apt + wslot * (3 * TSZ) + 2 * TSZ, traw);
    f32x4 U[4], dU[4], dW[4], W[4], dO[4];
    const int64_t e0 = (row0c * H + h) * kDim + col;
    {
        const int64_t pb = (row0c * H + h) * kDim;
        const uint32_t prs = static_cast<uint32_t>(rs);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            W[m] = unpark4(a.dk + pb, prs, m, g, col, L);
            dU[m] = unpark4(a.dla + pb, prs, m, g, col, L);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 16 * m + 4 * g + x;
                dO[m][x] = a.d_o[e0 + (r < L ? r : 0) * rs];
            }
        }
    }
    // this lane's row cw = col of S0 and dS1, columns 32 s + 8 g .. + 7
    float4 s0r[8], dsr[8];
    {
        const float* s0 = a.ws_s0 + wslot * SS + col * kDim;
        const float* ds = a.ws_ds + wslot * SS + col * kDim;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int j0 = 32 * s + 8 * g;
            s0r[2 * s] = *reinterpret_cast<const float4*>(s0 + j0);
            s0r[2 * s + 1] = *reinterpret_cast<const float4*>(s0 + j0 + 4);
            dsr[2 * s] = *reinterpret_cast<const float4*>(ds + j0);
            dsr[2 * s + 1] = *reinterpret_cast<const float4*>(ds + j0 + 4);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int x = 0; x < 4; ++x)
            if (16 * m + 4 * g + x >= L) W[m][x] = dU[m][x] = dO[m][x] = 0.f;

    // ---- staging: G and beta; k and q (bf16) and the images of T and T^T
    // into the image region, which is free until the phase B images
    __bf16* Kb = reinterpret_cast<__bf16*>(img + OFF_I2);
    __bf16* Qb = Kb + CH * kDim;
    constexpr int T_PL = CH * CH * 2;
    char* TIm = img + OFF_I0;            // T: rows r, k = i
    char* TTm = img + OFF_I0 + 2 * T_PL; // T^T: rows i, k = r
    tile_put<true, SEQ_NT>(traw, TTm);
    {
        // the same pieces as rows r = 2p, 2p + 1 of T, k = 4 (t mod 16) .. +3
        const int r = 2 * (t >> 4), i = 4 * (t & 15);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            img_put2<true>(TIm, T_PL, r + j, i, 2, traw.x[j].x, traw.x[j].y);
            img_put2<true>(TIm, T_PL, r + j, i + 2, 2, traw.x[j].z, traw.x[j].w);
        }
    }
    {
        Staged<SEQ_NT> st;
        stage_raw<SEQ_NT, true>(raw, tot, st);
        if (t < CH) bs[t] = t < L ? widen(braw) : 0.f;
#pragma unroll
        for (int j = 0; j < Staged<SEQ_NT>::TOK; ++j) {
            const int r = st.r0 + j;
            *reinterpret_cast<float2*>(&Gs[r * GLD + st.c0]) = make_float2(st.g[j][0], st.g[j][1]);
            *reinterpret_cast<uint32_t*>(&Kb[r * kDim + st.c0]) = raw.k[j];
            *reinterpret_cast<uint32_t*>(&Qb[r * kDim + st.c0]) = raw.q[j];
        }
        if (st.r0 == 0) {
            gLs[st.c0] = st.gl[0];
            gLs[st.c0 + 1] = st.gl[1];
        }
    }
    lds_sync();   // G, beta, k, q and the images of T
    // U = T (B W) and dW' = T^T dU (sums over tokens, 2 steps each)
#pragma unroll
    for (int m = 0; m < 4; ++m) U[m] = dW[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        f32x4 b0, b1;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            b0[x] = bs[16 * (2 * s) + 4 * g + x] * W[2 * s][x];
            b1[x] = bs[16 * (2 * s + 1) + 4 * g + x] * W[2 * s + 1][x];
        }
        bf16x8 wh, wl, uh, ul;
        bfrag(b0, b1, wh, wl);
        bfrag(dU[2 * s], dU[2 * s + 1], uh, ul);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            bf16x8 ah, al;
            img_frag(TIm, T_PL, m * 2 + s, lane, ah, al);
            U[m] = mma3(ah, al, wh, wl, U[m]);
            img_frag(TTm, T_PL, m * 2 + s, lane, ah, al);
            dW[m] = mma3(ah, al, uh, ul, dW[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int x = 0; x < 4; ++x)
            if (16 * m + 4 * g + x >= L) U[m][x] = dW[m][x] = 0.f;
    // queries and keys of this lane's rows and channel (read before the
    // barrier after which the images overwrite them)
    float qv[4][4], kv[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = 16 * m + 4 * g + x;
            qv[m][x] = (float)Qb[r * kDim + col];
            kv[m][x] = (float)Kb[r * kDim + col];
        }
    {
        // db (first term): row sums of dW' (.) W over this wave's columns
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 16 * m + 4 * g + x;
                const float p = row_sum16(dW[m][x] * W[m][x]);
                const float d = row_sum16(dO[m][x] * U[m][x]);  // the diagonal of dP in fp32
                if (l16 == 0) {
                    dbr[wave][r] = p;
                    dpd[wave][r] = d;
                }
            }
    }
    lds_sync();
    // dv = B dW'
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = 16 * m + 4 * g + x;
            if (r < L) a.dv[e0 + r * rs] = bs[r] * dW[m][x];
        }

    // ---- phase B images (natural binding, rows = tokens, k = value columns):
    // dO, -B dW', U.  An image element pair is two neighbouring columns held
    // by the lanes col and col ^ 1 (l16 even / odd): of the four rows 4g + x
    // of row block m, the even lane stores rows x = 0, 1 and the odd lane rows
    // x = 2, 3, each after taking the neighbour's two values (DPP).
    const bool even = (l16 & 1) == 0;
    const int kc = col & ~1;
    auto put_quad = [&](int off, int m, f32x4 v) {
        const float s0 = dpp_mov<kDppSwap1>(even ? v[2] : v[0]);
        const float s1 = dpp_mov<kDppSwap1>(even ? v[3] : v[1]);
        const int ra = 16 * m + 4 * g + (even ? 0 : 2);
        img_put2<false>(img + off, KT_PL, ra, kc, 4, even ? v[0] : s0, even ? s0 : v[2]);
        img_put2<false>(img + off, KT_PL, ra + 1, kc, 4, even ? v[1] : s1, even ? s1 : v[3]);
    };
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        f32x4 nw;
#pragma unroll
        for (int x = 0; x < 4; ++x) nw[x] = -bs[16 * m + 4 * g + x] * dW[m][x];
        put_quad(OFF_I0, m, dO[m]);
        put_quad(OFF_I1, m, nw);
        put_quad(OFF_I2, m, U[m]);
    }
    lds_sync();

    // ---- phase B: wave w on channels cw = 16w + l16; rows of S0 and dS1 as B operands
    {
        const int cw = col;
        bf16x8 sh[4], sl[4], dh[4], dl[4];
        float dg = 0.f;
        {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float4 a0 = s0r[2 * s], a1 = s0r[2 * s + 1];
                const float4 b0 = dsr[2 * s], b1 = dsr[2 * s + 1];
                const float xs[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                const float xd[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) dg += xs[j] * xd[j];
                split8(xs, sh[s], sl[s]);
                split8(xd, dh[s], dl[s]);
            }
            dg += __shfl_xor(dg, 16);
            dg += __shfl_xor(dg, 32);
        }
        const float gLc = gLs[cw];
        // per row: Qt dQt + Kt dKt (av) and Ke dKe (bv), channel cw
        float av[4][4], bv[4][4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 dQt = {0.f, 0.f, 0.f, 0.f}, dKt = dQt, dKe = dQt;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 ah, al;
                img_frag(img + OFF_I0, KT_PL, m * 4 + s, lane, ah, al);
                dQt = mma3(ah, al, sh[s], sl[s], dQt);
                img_frag(img + OFF_I1, KT_PL, m * 4 + s, lane, ah, al);
                dKt = mma3(ah, al, sh[s], sl[s], dKt);
                img_frag(img + OFF_I2, KT_PL, m * 4 + s, lane, ah, al);
                dKe = mma3(ah, al, dh[s], dl[s], dKe);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 16 * m + 4 * g + x;
                const float G = Gs[r * GLD + cw];
                const float gam = ex2(G), ge = ex2(gLc - G);
                const float q1 = qv[m][x], k1 = kv[m][x];
                const float dq = dQt[x] * gam;
                const float dkt = dKt[x] * gam, dke = dKe[x] * ge;
                const bool in = r < L;
                pp.q[m][x] = dq;
                pp.k[m][x] = dkt + dke;
                av[m][x] = in ? q1 * dq + k1 * dkt : 0.f;
                bv[m][x] = in ? k1 * dke : 0.f;
            }
        }
        // The S0 part of d log a_j: sum_{r >= j} av_r + sum_{r < j} bv_r +
        // gam_L dgam_L (suffix and prefix sums over the chunk's rows, held
        // by the four lane groups g in blocks of 16: each term is as small as
        // the decay it carries, with no cancellation between partial sums).
        float pre_prev = 0.f;   // bv over the blocks before m
        float sa_blk[4], sb_blk[4], sa_lane[4][4], sb_lane[4][4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float la_ = av[m][0] + av[m][1] + av[m][2] + av[m][3];
            const float lb_ = bv[m][0] + bv[m][1] + bv[m][2] + bv[m][3];
            sa_blk[m] = sb_blk[m] = 0.f;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                sa_lane[m][gg] = __shfl(la_, l16 + 16 * gg);
                sb_lane[m][gg] = __shfl(lb_, l16 + 16 * gg);
                sa_blk[m] += sa_lane[m][gg];
                sb_blk[m] += sb_lane[m][gg];
            }
        }
        const float glast = ex2(gLc) * dg;
        float after[4];
        after[3] = 0.f;
#pragma unroll
        for (int m = 2; m >= 0; --m) after[m] = after[m + 1] + sa_blk[m + 1];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float sa = after[m], sb = pre_prev;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                if (gg > g) sa += sa_lane[m][gg];
                if (gg < g) sb += sb_lane[m][gg];
            }
            // within this lane's four rows: suffix of av from x, prefix of bv before x
            float suf[4];
            suf[3] = sa + av[m][3];
#pragma unroll
            for (int x = 2; x >= 0; --x) suf[x] = suf[x + 1] + av[m][x];
            float run_b = sb;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                pp.l[m][x] = suf[x] + run_b + glast;
                run_b += bv[m][x];
            }
            pre_prev += sb_blk[m];
        }
    }
    // dP = dO U^T on the 10 lower 16 x 16 blocks (2 per wave for waves 0, 1),
    // zero above the diagonal inside the diagonal blocks
    for (int b = wave; b < 10; b += SEQ_NT / 64) {
        int mr = 0;
        while ((mr + 1) * (mr + 2) / 2 <= b) ++mr;
        const int mi = b - mr * (mr + 1) / 2;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 ah, al, bh2, bl2;
            img_frag(img + OFF_I0, KT_PL, mr * 4 + s, lane, ah, al);
            img_frag(img + OFF_I2, KT_PL, mi * 4 + s, lane, bh2, bl2);
            acc = mma3(ah, al, bh2, bl2, acc);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = 16 * mr + 4 * g + x, i = 16 * mi + l16;
            Pd[r * PLD + i] = i <= r ? acc[x] : 0.f;
        }
    }
    lds_sync();  // phase B images are dead
    // the intra-chunk part's independent inputs, in flight during phase C
    intra_request(a, id, h, row0c, L, rq);
    // dP_rr = dO_r . U_r carries the first token of a sequence from a zero
    // state (dq = dP_rr k_r there); its sum can cancel far below its terms, so
    // it is summed in fp32 rather than on split bf16
    if (t < CH) {
        float d = 0.f;
#pragma unroll
        for (int w = 0; w < SEQ_NT / 64; ++w) d += dpd[w][t];
        Pd[t * PLD + t] = d;
    }

    // ---- phase C: images of dU and B W, then dT = dU (B W)^T on the lower blocks
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        f32x4 bw;
#pragma unroll
        for (int x = 0; x < 4; ++x) bw[x] = bs[16 * m + 4 * g + x] * W[m][x];
        put_quad(OFF_I0, m, dU[m]);
        put_quad(OFF_I1, m, bw);
    }
    lds_sync();
    // dT (i < r) into LDS over the image of U, zero elsewhere: the 10 lower
    // blocks from the products, the 6 upper ones as zeros
    for (int b = wave; b < 10; b += SEQ_NT / 64) {
        int mr = 0;
        while ((mr + 1) * (mr + 2) / 2 <= b) ++mr;
        const int mi = b - mr * (mr + 1) / 2;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 ah, al, bh2, bl2;
            img_frag(img + OFF_I0, KT_PL, mr * 4 + s, lane, ah, al);
            img_frag(img + OFF_I1, KT_PL, mi * 4 + s, lane, bh2, bl2);
            acc = mma3(ah, al, bh2, bl2, acc);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = 16 * mr + 4 * g + x, i = 16 * mi + l16;
            Dt[r * PLD + i] = i < r ? acc[x] : 0.f;
        }
    }
#pragma unroll
    for (int e = t; e < 6 * 256; e += SEQ_NT) {
        int R, I;
        offdiag_block(e >> 8, R, I);   // (R, I) below the diagonal; (I, R) above it
        Dt[(16 * I + ((e >> 4) & 15)) * PLD + 16 * R + (e & 15)] = 0.f;
    }
    // db, first term
    if (t < L) {
        float sdb = 0.f;
#pragma unroll
        for (int w = 0; w < SEQ_NT / 64; ++w) sdb += dbr[w][t];
        a.dbeta[(row0c + t) * H + h] = sdb;
    }
}

// ================================================================ grads: intra-chunk part
//
// Per chunk of one head (512 threads; the second part of the grads kernel).
// Phase 1 (on split-bf16 matrix instructions):  dM = -T^T dT T^T,  dA = B dM (i < r),  db_r += sum_{i<r} dM_ri A_ri.
// Phase 2, wave w on channels 16w..16w+15: the decay products of dP and dA,
//   dq_r  = sum_{i<=r} dP_ri k_i 2^(G_r - G_i),   dk_r += sum_{i<r} dA_ri k_i 2^(G_r - G_i),
//   dk_i += sum_{r>=i} (dP_ri q_r + dA_ri k_r) 2^(G_r - G_i),
// on 16x16x16 matrix instructions per pair of 16-token blocks (R, I <= R),
// with 2^(G_r - G_i) = 2^(G_r - rho) 2^(rho - G_i).  For I < R, rho = G at the
// last token of block R - 1 and both factors are <= 1.  For I = R, rho = G at
// the block's 8th token, and a channel is taken this way only if both factors
// stay within 2^96; the others ("unsafe" channels, whose decay over half a
// block exceeds 2^-96) get that block pairwise on the vector ALUs.  Then dL,
// its reverse cumulative sum over the chunk, and the totals of dq and dk.

// LDS of the intra-chunk part.  dP, dT and G are where the gradient part left
// them; everything else overlays the gradient part's dead regions.
// k and q are kept channel-major (row stride KLD tokens), so that the rows a
// lane reads for its channel are contiguous.
// Phase 2 reads dP and dA as split-bf16 fragments formed once per workgroup
// (4 per pair of blocks (R, I <= R): rows of dP, rows of dA, columns of dP,
// columns of dA; 16 bytes per lane: high pair, low pair), the first NFR0 of
// them where T and A were, the rest where the gradient part's row sums were;
// the diagonal blocks also in fp32 (block stride DGB floats), and the cross
// sums of the diagonal blocks (16 slots of INTRA_NT) where dA and dP were.
constexpr int KLD = CH + 8;
constexpr int NFR = 4 * 10;
constexpr int NFR0 = 2 * CH * PLD * 4 / (64 * 16);
constexpr int DGB = 16 * 16 + 16;   // (+16: the four blocks start on different banks)
struct IntraLds {
    float U1[2 * CH * PLD];   // T and A, then (phase 2) fragments 0 .. NFR0 - 1
    __bf16 Ks[kDim * KLD];
    __bf16 Qs[kDim * KLD];
    float bs[CH], db2[CH];
    float Dg[2][4 * DGB];     // (phase 2) the diagonal blocks of dP and dA
    float Ad[CH * PLD];       // dT, Y, dM, dA, then (phase 2) cross sums, slots 0..7
    float Gs[CH * GLD];       // G (the gradient part's tile)
    uint4 Fr1[(NFR - NFR0) * 64];   // fragments NFR0 ..
    char pad1[offsetof(GradsLds, Pd) - offsetof(GradsLds, Gs) - CH * GLD * 4 - (NFR - NFR0) * 64 * 16];
    float Pd[CH * PLD];       // dP (i <= r), then (phase 2) cross sums, slots 8..15
};
static_assert(offsetof(IntraLds, Ad) == GR_DT_OFF, "dT where the gradient part wrote it");
static_assert(offsetof(IntraLds, Gs) == offsetof(GradsLds, Gs), "G where the gradient part staged it");
static_assert(offsetof(IntraLds, Pd) == offsetof(GradsLds, Pd), "dP where the gradient part wrote it");
static_assert(NFR0 * 64 * 16 == sizeof(IntraLds::U1), "whole fragments where T and A were");
static_assert(8 * INTRA_NT <= CH * PLD, "eight slots of cross sums fit in each of dA and dP");
static_assert(NFR % (INTRA_NT / 64) == 0, "the waves form the fragments in whole rounds");

__device__ __forceinline__ void intra_part(const ChunkBwdArgs& a, char* sm, IntraReq& rq, const Partials& pp)
{
    IntraLds& S_ = *reinterpret_cast<IntraLds*>(sm);
    float* Pd = S_.Pd;
    float* Ad = S_.Ad;
    float* U1 = S_.U1;
    __bf16* Ks = S_.Ks;
    __bf16* Qs = S_.Qs;
    float* bs = S_.bs;
    float* db2 = S_.db2;
    const float* Gs = S_.Gs;
    float* Ts = U1;
    float* As = U1 + CH * PLD;
    // phase 2: fragment f of the split dP and dA, and the cross sums' slot s
    auto frag = [&](int f) { return f < NFR0 ? reinterpret_cast<uint4*>(U1) + 64 * f : S_.Fr1 + 64 * (f - NFR0); };
    auto slot = [&](int s) { return s < 8 ? Ad + s * INTRA_NT : Pd + (s - 8) * INTRA_NT; };

    const int H = a.H;
    const int64_t id = blockIdx.x / H;
    const int h = static_cast<int>(blockIdx.x - id * H);
    int64_t n, c;
    if (!locate(a, id, n, c)) return;
    const int64_t row0c = seq_row0(a, n) + c * CH;
    const int L = static_cast<int>(min<int64_t>(CH, seq_len(a, n) - c * CH));
    const int t = threadIdx.x, lane = t & 63, wave = wave_id(), g = lane >> 4, l16 = lane & 15;

    // ---- dP, dT and G are in LDS (from the gradient part); the A and T
    // tiles were requested during the gradient part, k, q and beta kept from
    // its staging (rq)
    constexpr int NE = IntraReq::NE;
    const f32x4 (&ar)[NE] = rq.ar;
    const f32x4 (&tr)[NE] = rq.tr;
    const bf16_t braw = rq.braw;
    const ChunkRaw<INTRA_NT, true>& raw = rq.raw;
    // channel cc = 16 w + l16 of the rows 16 R + 4 g + x (as the gradient part's terms)
    const int cc = 16 * wave + l16;
    const int64_t rs = static_cast<int64_t>(H) * kDim;
    const int64_t e0 = (row0c * H + h) * kDim + cc;
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 1: T and A; k and q for phase 2 (the gradient part's
    // staging mapping: channels 2 (t mod 64), +1 of tokens TOK (t / 64) ..)
#pragma unroll
    for (int j = 0; j < NE; ++j) {
        const int e = t + j * INTRA_NT, r = e >> 4, i = 4 * (e & 15);
        *reinterpret_cast<f32x4*>(&As[r * PLD + i]) = ar[j];
        *reinterpret_cast<f32x4*>(&Ts[r * PLD + i]) = tr[j];
    }
    {
        constexpr int TOK = Staged<INTRA_NT>::TOK;
        const int c0 = 2 * (t & 63), r0 = TOK * wave;
        // (pairs of tokens per channel: the raw pairs hold two channels of one token)
#pragma unroll
        for (int j = 0; j < TOK; j += 2) {
            const uint32_t k0 = raw.k[j], k1 = raw.k[j + 1], q0 = raw.q[j], q1 = raw.q[j + 1];
            *reinterpret_cast<uint32_t*>(&Ks[c0 * KLD + r0 + j]) = (k0 & 0xffffu) | (k1 << 16);
            *reinterpret_cast<uint32_t*>(&Ks[(c0 + 1) * KLD + r0 + j]) = (k0 >> 16) | (k1 & 0xffff0000u);
            *reinterpret_cast<uint32_t*>(&Qs[c0 * KLD + r0 + j]) = (q0 & 0xffffu) | (q1 << 16);
            *reinterpret_cast<uint32_t*>(&Qs[(c0 + 1) * KLD + r0 + j]) = (q0 >> 16) | (q1 & 0xffff0000u);
        }
    }
    if (t < CH) bs[t] = t < L ? widen(braw) : 0.f;
    lds_sync();
    {
        // Y = T^T dT (Y_im = sum_r T_ri dT_rm) on split-bf16 16x16x32 matrix
        // instructions: wave w forms the tiles (I, M0) and (I, M0 + 1) with
        // I = w / 2, M0 = 2 (w mod 2); the operands are read from the fp32
        // tiles (T^T by columns of T, dT by columns), k = r.
        const int I = wave >> 1, M0 = 2 * (wave & 1);
        f32x4 y0 = {0.f, 0.f, 0.f, 0.f}, y1 = y0;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            float ta[8], b0[8], b1[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 32 * ks + 8 * g + j;
                ta[j] = Ts[r * PLD + 16 * I + l16];
                b0[j] = Ad[r * PLD + 16 * M0 + l16];
                b1[j] = Ad[r * PLD + 16 * M0 + 16 + l16];
            }
            bf16x8 ah, al, bh, bl;
            split8(ta, ah, al);
            split8(b0, bh, bl);
            y0 = mma3(ah, al, bh, bl, y0);
            split8(b1, bh, bl);
            y1 = mma3(ah, al, bh, bl, y1);
        }
        lds_sync();
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int i = 16 * I + 4 * g + x;
            Ad[i * PLD + 16 * M0 + l16] = y0[x];
            Ad[i * PLD + 16 * M0 + 16 + l16] = y1[x];
        }
    }
    lds_sync();
    {
        // dM = -Y T^T (dM_ik = -sum_m Y_im T_km; only k < i is used later), the
        // same tiling with (I, K0) and (I, K0 + 1): A = rows of Y, B = rows of T
        const int I = wave >> 1, K0 = 2 * (wave & 1);
        f32x4 m0 = {0.f, 0.f, 0.f, 0.f}, m1 = m0;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int c = 32 * ks + 8 * g;
            const f32x4* ya = reinterpret_cast<const f32x4*>(&Ad[(16 * I + l16) * PLD + c]);
            const f32x4* t0 = reinterpret_cast<const f32x4*>(&Ts[(16 * K0 + l16) * PLD + c]);
            const f32x4* t1 = reinterpret_cast<const f32x4*>(&Ts[(16 * K0 + 16 + l16) * PLD + c]);
            bf16x8 ah, al, bh, bl;
            bfrag(ya[0], ya[1], ah, al);
            bfrag(t0[0], t0[1], bh, bl);
            m0 = mma3(ah, al, bh, bl, m0);
            bfrag(t1[0], t1[1], bh, bl);
            m1 = mma3(ah, al, bh, bl, m1);
        }
        lds_sync();
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int i = 16 * I + 4 * g + x;
            Ad[i * PLD + 16 * K0 + l16] = -m0[x];
            Ad[i * PLD + 16 * K0 + 16 + l16] = -m1[x];
        }
    }
    lds_sync();
    {
        // db_r (second term): 8 threads per row, 8 columns each, then their sum
        const int r = t >> 3, k0 = 8 * (t & 7);
        float s2 = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) s2 += k0 + k < r ? Ad[r * PLD + k0 + k] * As[r * PLD + k0 + k] : 0.f;
        s2 = group_sum8(s2);
        if ((t & 7) == 0) db2[r] = s2;
    }
    lds_sync();
    for (int e = t; e < TSZ; e += INTRA_NT) {
        const int r = e >> 6, i = e & 63;
        Ad[r * PLD + i] = i < r ? bs[r] * Ad[r * PLD + i] : 0.f;   // dA
    }
    lds_sync();
    // ---- the operands of phase 2, split once for all waves (T and A are
    // dead): wave w forms the fragments w, w + 8, ..; fragment 4 p + m of the
    // p-th pair of blocks (R, I <= R) in the order (0,0), (1,0), (1,1), (2,0) ..
    // holds, for lane (g, l16), m = 0, 1: dP, dA at row 16 R + l16, columns
    // 16 I + 4 g ..; m = 2, 3: dP, dA at rows 16 R + 4 g .., column 16 I + l16
#pragma unroll
    for (int j = 0; j < NFR / (INTRA_NT / 64); ++j) {
        const int f = wave + (INTRA_NT / 64) * j, p = f >> 2, m = f & 3;
        const int R = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3, I = p - R * (R + 1) / 2;
        const float* src = (m & 1) ? Ad : Pd;
        float v[4];
        if (m < 2) {
            const float4 w = *reinterpret_cast<const float4*>(&src[(16 * R + l16) * PLD + 16 * I + 4 * g]);
            v[0] = w.x, v[1] = w.y, v[2] = w.z, v[3] = w.w;
        } else {
#pragma unroll
            for (int x = 0; x < 4; ++x) v[x] = src[(16 * R + 4 * g + x) * PLD + 16 * I + l16];
        }
        i16x4 hi, lo;
        split4(v[0], v[1], v[2], v[3], hi, lo);
        const uint2 h2 = __builtin_bit_cast(uint2, hi), l2 = __builtin_bit_cast(uint2, lo);
        frag(f)[lane] = (uint4){h2.x, h2.y, l2.x, l2.y};
    }
    {
        // the diagonal blocks in fp32: thread t takes 4 values of one row
        static_assert(INTRA_NT == 2 * 4 * 16 * 4, "one float4 per thread");
        const int m = t >> 8, R = (t >> 6) & 3, rl = (t >> 2) & 15, c4 = 4 * (t & 3);
        const float* src = m ? Ad : Pd;
        *reinterpret_cast<float4*>(&S_.Dg[m][R * DGB + 16 * rl + c4]) =
            *reinterpret_cast<const float4*>(&src[(16 * R + rl) * PLD + 16 * R + c4]);
    }
    lds_sync();   // dP and dA are read: the cross sums take their place
    const float* DgP = S_.Dg[0];
    const float* DgA = S_.Dg[1];

    // ---- phase 2: wave w on channels cc = 16w + l16; rows 16R + 4g + x of each block R
    auto Gv = [&](int r) { return Gs[r * GLD + cc]; };
    auto Kv = [&](int r) { return (float)Ks[cc * KLD + r]; };
    auto Qv = [&](int r) { return (float)Qs[cc * KLD + r]; };
    // The cross sums C_j = sum_{r >= j > i} X_ri of the decay products
    // X_ri = (dA_ri k_r + dP_ri q_r) k_i 2^(G_r - G_i) (this lane's channel)
    // are the A/P part of d log a_j.  By blocks, for j in block J: Ab[J] the
    // blocks entirely after and before J, Bc[J] the column sums over the row
    // blocks after J (columns in J), the row sums over the column blocks
    // before J (rows in J), and the pairs inside J (explicit).  Every term
    // carries the decay over token j.  Row blocks run last to first, so that
    // a block's dk column sums, Bc and Ab are complete when it is written.
    // The pairs inside each diagonal block first, into the slots: lane group g takes
    // the diagonal block R = g of channel cc, all 16 of its rows (no lane
    // computes a pair above the diagonal, and no sum crosses lanes).  With
    // a_r = k_r 2^(G_r - rho), c_r = q_r 2^(G_r - rho), b_i = k_i 2^(rho - G_i),
    // X_ri = (dA_ri a_r + dP_ri c_r) b_i; cs[j] gathers, over the rows r >= j,
    // the row sums over the columns i < j.
    __builtin_amdgcn_sched_barrier(0);
    {
        const int R = g, r0 = 16 * g;
        const float rho = Gv(r0 + 7);
        const bool safe = Gv(r0) - rho <= 96.f && rho - Gv(r0 + 15) <= 96.f;
        float bcol[16], cs[16];
        // (values formed unconditionally and then selected: an LDS read under
        // the condition would become a branch of its own)
#pragma unroll
        for (int il = 0; il < 16; ++il) {
            const float b = Kv(r0 + il) * ex2(rho - Gv(r0 + il));
            bcol[il] = safe ? b : 0.f;
            cs[il] = 0.f;
        }
        // rows last to first: col[i] is the sum of dA_ri a_r + dP_ri c_r over
        // the rows r >= rl taken so far, so that cs[rl] = sum_{i < rl} b_i col[i]
        float colv[15];
#pragma unroll
        for (int il = 0; il < 15; ++il) colv[il] = 0.f;
#pragma unroll
        for (int rl = 15; rl >= 1; --rl) {
            const int r = r0 + rl;
            const float e = ex2(Gv(r) - rho);
            const float f = safe ? e : 0.f;
            const float ar = Kv(r) * f, cr = Qv(r) * f;
            const float* da = &DgA[R * DGB + 16 * rl];
            const float* dp = &DgP[R * DGB + 16 * rl];
            float acc = 0.f;
#pragma unroll
            for (int il = 0; il < rl; ++il) {
                colv[il] = fmaf(da[il], ar, colv[il]);
                colv[il] = fmaf(dp[il], cr, colv[il]);
                acc = fmaf(bcol[il], colv[il], acc);
            }
            cs[rl] = acc;
            __builtin_amdgcn_sched_barrier(0);   // one row at a time: bounded register use
        }
        if (__any(!safe)) {
            // the unsafe channels' pairs, with pairwise factors
            if (!safe) {
                for (int rl = 1; rl < 16; ++rl) {
                    const int r = r0 + rl;
                    const float gr = Gv(r), kr = Kv(r), qr = Qv(r);
                    float run = 0.f;
#pragma unroll
                    for (int il = 0; il < 15; ++il) {
                        if (il < rl) {
                            const int i = r0 + il;
                            run += (DgA[R * DGB + 16 * rl + il] * kr + DgP[R * DGB + 16 * rl + il] * qr) * Kv(i) * ex2(gr - Gv(i));
                            cs[il + 1] += run;
                        }
                    }
                }
            }
        }
        // to the thread that finalises row j = 16 R + jl: lane group jl / 4, slot 4 R + jl mod 4
        float* dgs = g < 2 ? Ad + 4 * g * INTRA_NT : Pd + (4 * g - 8) * INTRA_NT;   // slots 4 R ..
#pragma unroll
        for (int jl = 0; jl < 16; ++jl)
            dgs[(jl & 3) * INTRA_NT + 64 * wave + 16 * (jl >> 2) + l16] = cs[jl];
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 dkc[4];
    float Bc[4][4], Ab[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        dkc[R] = (f32x4){0.f, 0.f, 0.f, 0.f};
        Ab[R] = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) Bc[R][x] = 0.f;
    }
#pragma unroll
    for (int R = 3; R >= 0; --R) {
        float gR[4], kR[4], qR[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            gR[x] = Gv(16 * R + 4 * g + x);
            kR[x] = Kv(16 * R + 4 * g + x);
            qR[x] = Qv(16 * R + 4 * g + x);
        }
        f32x4 dqR = {0.f, 0.f, 0.f, 0.f}, dkrR = dqR;
        float Cr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int I = 0; I <= R; ++I) {
            const float rho = I < R ? Gv(16 * R - 1) : Gv(16 * R + 7);
            const bool safe = I < R || (Gv(16 * R) - rho <= 96.f && rho - Gv(16 * R + 15) <= 96.f);
            float f[4], hh[4], kI[4], kh[4], qf[4], kf[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int i = 16 * I + 4 * g + x;
                const float fe = ex2(gR[x] - rho), he = ex2(rho - Gv(i));
                f[x] = safe ? fe : 0.f;
                hh[x] = safe ? he : 0.f;
                kI[x] = Kv(i);
                kh[x] = kI[x] * hh[x];
                qf[x] = qR[x] * f[x];
                kf[x] = kR[x] * f[x];
            }
            i16x4 bkh, bkl, bqh, bql, bfh, bfl;
            split4(kh[0], kh[1], kh[2], kh[3], bkh, bkl);
            split4(qf[0], qf[1], qf[2], qf[3], bqh, bql);
            split4(kf[0], kf[1], kf[2], kf[3], bfh, bfl);
            // row side: A = dP_RI, dA_RI (row l16 of block R, columns 4g.. of block I)
            const int f0 = 4 * (R * (R + 1) / 2 + I);
            const uint4 frp = frag(f0)[lane], fra = frag(f0 + 1)[lane];
            const uint4 fcp = frag(f0 + 2)[lane], fca = frag(f0 + 3)[lane];
            const i16x4 aph = __builtin_bit_cast(i16x4, (uint2){frp.x, frp.y});
            const i16x4 apl = __builtin_bit_cast(i16x4, (uint2){frp.z, frp.w});
            const i16x4 aah = __builtin_bit_cast(i16x4, (uint2){fra.x, fra.y});
            const i16x4 aal = __builtin_bit_cast(i16x4, (uint2){fra.z, fra.w});
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 sq = mma16(aph, apl, bkh, bkl, z);
            const f32x4 sk = mma16(aah, aal, bkh, bkl, z);
            // column side: A = dP_RI^T, dA_RI^T (row l16 of block I, columns 4g.. of block R)
            const i16x4 cph = __builtin_bit_cast(i16x4, (uint2){fcp.x, fcp.y});
            const i16x4 cpl = __builtin_bit_cast(i16x4, (uint2){fcp.z, fcp.w});
            const i16x4 cah = __builtin_bit_cast(i16x4, (uint2){fca.x, fca.y});
            const i16x4 cal = __builtin_bit_cast(i16x4, (uint2){fca.z, fca.w});
            f32x4 sc = mma16(cph, cpl, bqh, bql, z);
            sc = mma16(cah, cal, bfh, bfl, sc);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                dqR[x] += f[x] * sq[x];
                dkrR[x] += f[x] * sk[x];
                dkc[I][x] += hh[x] * sc[x];
            }
            if (I < R) {
                // an off-diagonal block: its row sums (rows in R), column sums
                // (columns in I) and, when some block J lies between, its total
                float tsum = 0.f;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float rx = f[x] * (qR[x] * sq[x] + kR[x] * sk[x]);
                    Cr[x] += rx;
                    tsum += rx;
                    Bc[I][x] += kI[x] * hh[x] * sc[x];
                }
                if (I + 1 < R) {
                    tsum += __shfl_xor(tsum, 16);
                    tsum += __shfl_xor(tsum, 32);
#pragma unroll
                    for (int J = I + 1; J < R; ++J) Ab[J] += tsum;
                }
            } else {
                if (__any(!safe)) {
                    // pairwise on the vector ALUs for the unsafe channels
                    if (!safe) {
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            const int r = 16 * R + 4 * g + x;
                            float aq = 0.f, ak = 0.f, acc = 0.f;
                            const int d = R * DGB, rl = 4 * g + x;   // the diagonal block, row rl
                            for (int i = 16 * R; i <= r; ++i) {
                                const float kie = Kv(i) * ex2(gR[x] - Gv(i));
                                aq += DgP[d + 16 * rl + i - 16 * R] * kie;
                                ak += DgA[d + 16 * rl + i - 16 * R] * kie;
                            }
                            const float gi = gR[x];  // row r as the column index i
                            for (int rr = r; rr < 16 * R + 16; ++rr)
                                acc += (DgP[d + 16 * (rr - 16 * R) + rl] * Qv(rr) + DgA[d + 16 * (rr - 16 * R) + rl] * Kv(rr)) *
                                       ex2(Gv(rr) - gi);
                            dqR[x] += aq;
                            dkrR[x] += ak;
                            dkc[R][x] += acc;
                        }
                    }
                }
            }
        }

        // ---- block R is complete: dq, dk and d log a of its rows, added to
        // the grads kernel's terms
        const float bl = Bc[R][0] + Bc[R][1] + Bc[R][2] + Bc[R][3];
        const float cl = Cr[0] + Cr[1] + Cr[2] + Cr[3];
        float bpre = 0.f, csuf = 0.f;   // over the lane groups before / after g
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const float bg = __shfl(bl, l16 + 16 * gg);
            const float cg = __shfl(cl, l16 + 16 * gg);
            if (gg < g) bpre += bg;
            if (gg > g) csuf += cg;
        }
        float cs[4];   // suffix of the row sums from x
        cs[3] = csuf + Cr[3];
#pragma unroll
        for (int x = 2; x >= 0; --x) cs[x] = cs[x + 1] + Cr[x];
        float bp = bpre;   // prefix of the column sums before x
        float fq[4], fk[4], fl[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            fq[x] = pp.q[R][x] + dqR[x];
            fk[x] = pp.k[R][x] + dkrR[x] + dkc[R][x];
            fl[x] = pp.l[R][x] + Ab[R] + bp + cs[x] + slot(4 * R + x)[t];
            bp += Bc[R][x];
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = 16 * R + 4 * g + x;
            if (r < L) {
                const int64_t e = e0 + r * rs;
                a.dq[e] = fq[x];
                a.dk[e] = fk[x];
                a.dla[e] = fl[x];
            }
        }
    }
    if (t < L) a.dbeta[(row0c + t) * H + h] += db2[t];
}

// The gradient part and then the intra-chunk part of one chunk of one head
// (grid: chunk ids x heads; 512 threads).  The intra part takes the partial
// dq, dk and d log alpha of the gradient part in registers and dP, dT from LDS
// (written by other waves, before the barrier).
constexpr size_t kGiLds = sizeof(GradsLds) > sizeof(IntraLds) ? sizeof(GradsLds) : sizeof(IntraLds);
static_assert(kGiLds <= 160 * 1024, "LDS budget of one CU");
static_assert(INTRA_NT == SEQ_NT, "one workgroup shape for both parts");

__global__ __launch_bounds__(SEQ_NT, 1) void chunk_grads_kernel(const ChunkBwdArgs a)
{
    __shared__ __attribute__((aligned(16))) char sm[kGiLds];
    IntraReq rq;
    Partials pp;
    grads_part(a, sm, rq, pp);
    __syncthreads();   // dP and dT complete; the rest of the LDS free
    intra_part(a, sm, rq, pp);
}

}  // namespace

// the workspace the plan sizes: entering state, leaving-state gradient and
// A/P/T, per (chunk id, head)
static_assert(kChunkBackwardFloats == 2 * static_cast<size_t>(SS) + 3 * TSZ,
              "the workspace layout of the chunked backward");
static_assert(CH == kChunk, "the plan's chunk length");

hipError_t launch_backward_chunked(const void* q, const void* k, const void* v, const void* beta,
                                   const float* log_alpha, const float* d_o, const int32_t* cu_seqlens,
                                   int64_t n_seq, int64_t T, int64_t H, const float* initial_state,
                                   const float* d_final_state, float* dq, float* dk, float* dv,
                                   float* dbeta, float* dlog_alpha, float* d_initial_state,
                                   int64_t n_ids, void* ws, hipStream_t stream)
{
    const int64_t units = n_seq * H;
    if (units <= 0) return hipSuccess;
    ChunkBwdArgs a = {};
    a.q = static_cast<const bf16_t*>(q);
    a.k = static_cast<const bf16_t*>(k);
    a.v = static_cast<const bf16_t*>(v);
    a.beta = static_cast<const bf16_t*>(beta);
    a.la = log_alpha;
    a.d_o = d_o;
    a.cu = cu_seqlens;
    a.T = T;
    a.n_seq = n_seq;
    a.H = static_cast<int>(H);
    a.s0 = initial_state;
    a.d_sT = d_final_state;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dbeta = dbeta;
    a.dla = dlog_alpha;
    a.ds0 = d_initial_state;
    const size_t slots = static_cast<size_t>(n_ids) * H;
    float* w = static_cast<float*>(ws);
    a.ws_s0 = w;
    a.ws_ds = a.ws_s0 + slots * SS;
    a.ws_apt = a.ws_ds + slots * SS;

    const dim3 chunks(static_cast<unsigned>(n_ids * H)), seqs(static_cast<unsigned>(units));
    hipError_t e;
    if (n_ids > 0) {
        hipLaunchKernelGGL(chunk_prep_kernel, chunks, dim3(PREP_NT), 0, stream, a);
        e = hipGetLastError();
        report("backward prep launch", e);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(chunk_states_kernel, seqs, dim3(SEQ_NT), 0, stream, a);
    e = hipGetLastError();
    report("backward states launch", e);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_dstate_kernel, seqs, dim3(SEQ_NT), 0, stream, a);
    e = hipGetLastError();
    report("backward state-gradient launch", e);
    if (e != hipSuccess || n_ids == 0) return e;
    hipLaunchKernelGGL(chunk_grads_kernel, chunks, dim3(SEQ_NT), 0, stream, a);
    e = hipGetLastError();
    report("backward gradient launch", e);
    return e;
}

}  // namespace kda
