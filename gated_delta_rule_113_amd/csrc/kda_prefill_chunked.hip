// Chunked (blockwise) KDA prefill on bf16 MFMA, fp32 state on chip.
//
// The recurrence (per head; S is d_k x d_v, rows = forgetting channels)
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t
// is evaluated 64 tokens at a time ("blockwise so it maps onto matrix units":
// "Kimi K3 -- the architecture and infrastructure, explained", section "Kimi
// Delta Attention: the load-bearing choice"; update rule from section "How the
// delta rule actually works", per-channel gate as in the same section).
// Within a chunk of tokens r = 0..63 entering with state S0, with G_r the
// inclusive cumulative log2-decay of each channel:
//     A_ri  = sum_c k_rc k_ic 2^(G_rc - G_ic)   (i < r)      key-key interactions
//     Pt_ir = sum_c q_rc k_ic 2^(G_rc - G_ic)   (i <= r)     query-key interactions
//     T     = (I + Diag(b) A)^-1                              (UT transform)
//     X     = Kt S0,   Kt_r = k_r * 2^G_r                      decayed keys
//     U     = T Diag(b) (V - X)                               corrected writes
//     O     = Qt S0 + P U,   Qt_r = q_r * 2^G_r
//     S1    = Diag(2^G_63) S0 + Ke^T U,   Ke_i = k_i * 2^(G_63 - G_i)
// which is the token recurrence regrouped (exact in real arithmetic).
//
// Overflow-free decay factors: 2^(G_r - G_i) is never formed from 2^(-G_i).
// Tiles of 16 x 16 tokens pair a row factor 2^(G_r - rho) with a column factor
// 2^(rho - G_i) for a per-row-block reference rho between i and r:
//  - off-diagonal tiles (row block rb > column block ib): the column factor is
//    2^(G_end(ib) - G_i) <= 1 times the per-channel scalar 2^(rho_rb - G_end(ib))
//    <= 1, so whichever piece underflows, the true product was below 2^-30;
//  - diagonal tiles use rho = G at the block's 8th token when every channel's
//    log2-decay from there to either end of the block is <= 96; both factors
//    are then formed directly and stay in [2^-96, 2^96].  Otherwise the block
//    takes rho = G at the end of the previous block (all off-diagonal factors
//    <= 1) and its diagonal tile is computed pairwise on the vector ALUs.
//
// Precision: every MFMA operand that is not an exact bf16 input is split into
// hi + lo bf16 parts and each product uses hi*hi + hi*lo + lo*hi with fp32
// accumulation (about 16 significant bits per operand); the state, decay
// factors, T and all accumulations are fp32.
//
// Work decomposition: one workgroup (4 waves) per (sequence, head, 16-column
// slice of d_v).  Columns of S evolve independently, so the 8 slices of a head
// run in parallel; each recomputes the d_v-independent part (A, P, T, factors).
// The 8 slices of a head are placed on one XCD so that they share its L2 for
// the q/k/log_alpha reads.  The state slice (128 x 16 fp32) lives in MFMA
// accumulators across chunks and is written to memory once at the end.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;            // tokens per chunk
constexpr int DVS = 16;           // value columns per workgroup
constexpr int NSLICE = kDim / DVS;
constexpr int QK_LD = kDim + 8;   // bf16 row stride of q/k/state^T tiles in LDS
constexpr int G_LD = kDim + 4;    // fp32 row stride of [64][128] tiles
constexpr int T_LD = CH + 4;      // fp32 row stride of [64][64] tiles
constexpr int Y_LD = CH + 8;      // bf16 row stride of [16][64] tiles
constexpr float kSafeLog2 = 96.f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void split1(float x, __bf16& h, __bf16& l)
{
    h = (__bf16)x;
    l = (__bf16)(x - (float)h);
}

__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& h, bf16x8& l)
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        __bf16 a, b;
        split1(x[j], a, b);
        h[j] = a;
        l[j] = b;
    }
}

__device__ __forceinline__ void split4(const float (&x)[4], bf16x4& h, bf16x4& l)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        __bf16 a, b;
        split1(x[j], a, b);
        h[j] = a;
        l[j] = b;
    }
}

// hi*hi + hi*lo + lo*hi on the 16x16x32 and 16x16x16 bf16 matrix instructions.
__device__ __forceinline__ f32x4 mma32x3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ f32x4 mma16x3(bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl, f32x4 c)
{
    const i16x4 AH = __builtin_bit_cast(i16x4, ah), AL = __builtin_bit_cast(i16x4, al);
    const i16x4 BH = __builtin_bit_cast(i16x4, bh), BL = __builtin_bit_cast(i16x4, bl);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(AL, BH, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(AH, BL, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(AH, BH, c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

struct Smem {
    __bf16 q[CH * QK_LD];            // raw bf16 queries of the chunk
    __bf16 k[CH * QK_LD];            // raw bf16 keys
    float g[CH * G_LD];              // log2-decay, then its cumulative sum G; later N
    float cb[CH * G_LD];             // k_i 2^(G_end(b(i)) - G_i)
    float scal[10 * kDim];           // 2^(rho_rb - G_end(ib)), tile t = rb(rb+1)/2 + ib < rb
    float kend[4 * kDim];            // 2^(G_63 - G_end(ib))
    float erho[4 * kDim];            // 2^(rho_rb)
    float rho[4 * kDim];             // rho_rb
    float el[kDim];                  // 2^(G_63)
    float beta[CH];
    float v[CH * DVS];               // value slice, fp32
    float t[CH * T_LD];              // T = (I + N)^-1
    __bf16 st[2][DVS * QK_LD];       // state^T slice, hi / lo   [j][channel]
    __bf16 y[2][DVS * Y_LD];         // Y^T = (b (V - X))^T,     [j][token]
    __bf16 u[2][DVS * Y_LD];         // U^T                      [j][token]
    int unsafe[4];
};

__global__ __launch_bounds__(256, 1) void prefill_chunked_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ beta, const float* __restrict__ log_alpha,
    const int32_t* __restrict__ cu_seqlens, int64_t T, int H, int64_t units,
    const float* initial_state, float* __restrict__ o, float* final_state)
{
    __shared__ Smem sm;
    float* const sN = sm.g;  // N = Diag(b) A reuses the G tile once G is consumed

    // workgroup -> (unit, slice); consecutive workgroups go to consecutive XCDs,
    // so unit u's slices all land on XCD u % 8.
    const int wg = blockIdx.x;
    const int slice = (wg >> 3) & (NSLICE - 1);
    const int64_t unit = static_cast<int64_t>(wg >> 6) * 8 + (wg & 7);
    if (unit >= units) return;
    const int64_t n = unit / H;
    const int h = static_cast<int>(unit - n * H);
    int64_t row0, len;
    if (cu_seqlens) {
        row0 = cu_seqlens[n];
        len = static_cast<int64_t>(cu_seqlens[n + 1]) - row0;
    } else {
        row0 = n * T;
        len = T;
    }

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;
    const int col0 = slice * DVS;

    // ---- state slice: wave w owns channel tiles 2w, 2w+1; lane holds
    //      S[16t + 4 g4 + i][col0 + l16], i = 0..3 (matrix-core accumulator layout)
    f32x4 sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int t = 2 * wave + tt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = 16 * t + 4 * g4 + i;
            sacc[tt][i] = initial_state
                              ? initial_state[unit * (kDim * kDim) + ch * kDim + col0 + l16]
                              : 0.f;
        }
    }
    auto store_state_t = [&]() {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * wave + tt;
            float x[4] = {sacc[tt][0], sacc[tt][1], sacc[tt][2], sacc[tt][3]};
            bf16x4 hi, lo;
            split4(x, hi, lo);
            *reinterpret_cast<bf16x4*>(&sm.st[0][l16 * QK_LD + 16 * t + 4 * g4]) = hi;
            *reinterpret_cast<bf16x4*>(&sm.st[1][l16 * QK_LD + 16 * t + 4 * g4]) = lo;
        }
    };
    store_state_t();

    // ---- prefetch registers for one chunk of inputs
    uint4 pq[4], pk[4];
    float4 pla[8];
    uint4 pv = make_uint4(0, 0, 0, 0);
    uint16_t pb = 0;
    auto prefetch = [&](int64_t c0, int64_t L) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int p = tid + 256 * m;
            const int tok = p >> 4, piece = p & 15;
            if (tok < L) {
                const int64_t off = ((row0 + c0 + tok) * H + h) * kDim + 8 * piece;
                pq[m] = *reinterpret_cast<const uint4*>(q + off);
                pk[m] = *reinterpret_cast<const uint4*>(k + off);
            } else {
                pq[m] = make_uint4(0, 0, 0, 0);
                pk[m] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int p = tid + 256 * m;
            const int tok = p >> 5, piece = p & 31;
            pla[m] = tok < L ? *reinterpret_cast<const float4*>(
                                   log_alpha + ((row0 + c0 + tok) * H + h) * kDim + 4 * piece)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (tid < 128) {
            const int tok = tid >> 1, half = tid & 1;
            pv = tok < L ? *reinterpret_cast<const uint4*>(
                               v + ((row0 + c0 + tok) * H + h) * kDim + col0 + 8 * half)
                         : make_uint4(0, 0, 0, 0);
        } else if (tid < 192) {
            const int tok = tid - 128;
            pb = tok < L ? beta[(row0 + c0 + tok) * H + h].bits : uint16_t(0);
        }
    };

    const int64_t nchunks = (len + CH - 1) / CH;
    if (nchunks > 0) prefetch(0, len < CH ? len : CH);

    for (int64_t ci = 0; ci < nchunks; ++ci) {
        const int64_t c0 = ci * CH;
        const int64_t L = (len - c0) < CH ? (len - c0) : CH;

        // ================= A: stage the chunk in LDS, prefetch the next =====
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int p = tid + 256 * m;
            const int tok = p >> 4, piece = p & 15;
            *reinterpret_cast<uint4*>(&sm.q[tok * QK_LD + 8 * piece]) = pq[m];
            *reinterpret_cast<uint4*>(&sm.k[tok * QK_LD + 8 * piece]) = pk[m];
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int p = tid + 256 * m;
            const int tok = p >> 5, piece = p & 31;
            float4 x = pla[m];
            x.x *= kLog2e; x.y *= kLog2e; x.z *= kLog2e; x.w *= kLog2e;
            *reinterpret_cast<float4*>(&sm.g[tok * G_LD + 4 * piece]) = x;
        }
        if (tid < 128) {
            const int tok = tid >> 1, half = tid & 1;
            const uint32_t w[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sm.v[tok * DVS + 8 * half + 2 * e] = __uint_as_float(w[e] << 16);
                sm.v[tok * DVS + 8 * half + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
            }
        } else if (tid < 192) {
            sm.beta[tid - 128] = bf(pb);
        }
        if (tid < 4) sm.unsafe[tid] = 0;
        if (ci + 1 < nchunks) {
            const int64_t c1 = c0 + CH;
            prefetch(c1, (len - c1) < CH ? (len - c1) : CH);
        }
        __syncthreads();

        // ================= B: cumulative decay, safety, factor tables ========
        {
            const int c = tid & 127, half = tid >> 7;
            float acc = 0.f;
            for (int r = 32 * half; r < 32 * half + 32; ++r) {
                acc += sm.g[r * G_LD + c];
                sm.g[r * G_LD + c] = acc;
            }
        }
        __syncthreads();
        if (tid >= 128) {
            const int c = tid & 127;
            const float base = sm.g[31 * G_LD + c];
            for (int r = 32; r < 64; ++r) sm.g[r * G_LD + c] += base;
        }
        __syncthreads();
        for (int e = tid; e < 4 * kDim; e += 256) {
            const int b = e >> 7, c = e & 127;
            const float gs = sm.g[(16 * b) * G_LD + c];
            const float gm = sm.g[(16 * b + 7) * G_LD + c];
            const float ge = sm.g[(16 * b + 15) * G_LD + c];
            if (gs - gm > kSafeLog2 || gm - ge > kSafeLog2) atomicOr(&sm.unsafe[b], 1);
        }
        __syncthreads();
        for (int e = tid; e < 4 * kDim; e += 256) {
            const int b = e >> 7, c = e & 127;
            float r;
            if (!sm.unsafe[b]) r = sm.g[(16 * b + 7) * G_LD + c];
            else r = b > 0 ? sm.g[(16 * b - 1) * G_LD + c] : 0.f;
            sm.rho[b * kDim + c] = r;
            sm.erho[b * kDim + c] = ex2(r);
            sm.kend[b * kDim + c] = ex2(sm.g[63 * G_LD + c] - sm.g[(16 * b + 15) * G_LD + c]);
        }
        if (tid < 128) sm.el[tid] = ex2(sm.g[63 * G_LD + tid]);
        __syncthreads();
        for (int e = tid; e < 10 * kDim; e += 256) {
            const int t = e >> 7, c = e & 127;
            const int rb = t >= 6 ? 3 : (t >= 3 ? 2 : (t >= 1 ? 1 : 0));
            const int ib = t - rb * (rb + 1) / 2;
            // off-diagonal tiles only (ib < rb): rho_rb <= G_end(ib), the factor is <= 1
            sm.scal[e] = ib < rb ? ex2(sm.rho[rb * kDim + c] - sm.g[(16 * ib + 15) * G_LD + c]) : 0.f;
        }
        for (int e = tid; e < CH * kDim; e += 256) {
            const int i = e >> 7, c = e & 127;
            const float ge = sm.g[((i & ~15) + 15) * G_LD + c];
            sm.cb[i * G_LD + c] =
                (float)sm.k[i * QK_LD + c] * ex2(ge - sm.g[i * G_LD + c]);
        }
        __syncthreads();

        // ================= C1: row fragments of row block rb = wave =========
        const int rb = wave;
        const int rrow = 16 * rb + l16;  // token of this lane in A-operand layout
        const bool unsafe_rb = sm.unsafe[rb] != 0;
        // fk/fq: row operands k_r 2^(G_r - rho), q_r 2^(G_r - rho) of this lane's
        // token; cd: the diagonal tile's column operand k_i 2^(rho - G_i) for the
        // same token (lane layout of a column operand is the same), taken
        // directly so that no factor of the tile leaves [2^-96, 2^96].
        bf16x8 fkh[4], fkl[4], fqh[4], fql[4], cdh[4], cdl[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c0s = 32 * s + 8 * g4;
            const bf16x8 kq = *reinterpret_cast<const bf16x8*>(&sm.k[rrow * QK_LD + c0s]);
            const bf16x8 qq = *reinterpret_cast<const bf16x8*>(&sm.q[rrow * QK_LD + c0s]);
            float xk[8], xq[8], xd[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float d = sm.g[rrow * G_LD + c0s + j] - sm.rho[rb * kDim + c0s + j];
                const float f = ex2(d);
                xk[j] = (float)kq[j] * f;
                xq[j] = (float)qq[j] * f;
                xd[j] = unsafe_rb ? 0.f : (float)kq[j] * ex2(-d);
            }
            split8(xk, fkh[s], fkl[s]);
            split8(xq, fqh[s], fql[s]);
            split8(xd, cdh[s], cdl[s]);
        }
        // Diagonal tile computed pairwise when the block's decay is too steep
        // for a single reference.  Lane layouts match the matrix-core results:
        //   a_d[i] = A[16rb + 4 g4 + i][16rb + l16],  pt_d[i] = Pt[16rb + 4 g4 + i][16rb + l16]
        f32x4 a_d = {0.f, 0.f, 0.f, 0.f}, pt_d = {0.f, 0.f, 0.f, 0.f};
        if (unsafe_rb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ra = 16 * rb + 4 * g4 + i;   // A: row token
                const int ia = 16 * rb + l16;          // A: column token
                float sa = 0.f, sp = 0.f;
                for (int c = 0; c < kDim; ++c) {
                    if (ra > ia)
                        sa += (float)sm.k[ra * QK_LD + c] * (float)sm.k[ia * QK_LD + c] *
                              ex2(sm.g[ra * G_LD + c] - sm.g[ia * G_LD + c]);
                    if (ra <= ia)   // Pt[i = ra][r = ia]: query row ia, key row ra
                        sp += (float)sm.q[ia * QK_LD + c] * (float)sm.k[ra * QK_LD + c] *
                              ex2(sm.g[ia * G_LD + c] - sm.g[ra * G_LD + c]);
                }
                a_d[i] = sa;
                pt_d[i] = sp;
            }
        }
        __syncthreads();  // G is dead from here on; its tile now holds N

        // ================= C2: A and P^T tiles of row block rb ==============
        bf16x4 pth[4], ptl[4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            if (ib > rb) break;
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
            if (ib == rb && unsafe_rb) {
                accA = a_d;
                accP = pt_d;
            } else {
                const int icol = 16 * ib + l16;  // token of this lane as a column
                const int t = rb * (rb + 1) / 2 + ib;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int c0s = 32 * s + 8 * g4;
                    bf16x8 ch, cl;
                    if (ib == rb) {
                        ch = cdh[s];
                        cl = cdl[s];
                    } else {
                        // k_i 2^(G_end(ib) - G_i) <= 1 times 2^(rho_rb - G_end(ib)) <= 1:
                        // a piece that underflows bounds a product below 2^-30
                        float x[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            x[j] = sm.cb[icol * G_LD + c0s + j] * sm.scal[t * kDim + c0s + j];
                        split8(x, ch, cl);
                    }
                    accA = mma32x3(fkh[s], fkl[s], ch, cl, accA);
                    accP = mma32x3(ch, cl, fqh[s], fql[s], accP);
                }
            }
            // N = Diag(beta) A, strictly lower
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rb + 4 * g4 + i, c = 16 * ib + l16;
                sN[r * T_LD + c] = (r > c) ? sm.beta[r] * accA[i] : 0.f;
            }
            // P^T tile as the B operand of U^T P^T: rows i = 16ib + 4 g4 + e, col r = rrow
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * ib + 4 * g4 + e;
                x[e] = (i <= rrow) ? accP[e] : 0.f;
            }
            split4(x, pth[ib], ptl[ib]);
        }
        __syncthreads();

        // ================= D: T = (I + N)^-1, blockwise ======================
        {
            // diagonal block b = wave by forward substitution; lane = (column jc, part p)
            const int b = wave, jc = lane >> 2, p = lane & 3;
            float tv[4] = {0.f, 0.f, 0.f, 0.f};  // T[16b + p + 4m][16b + jc]
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = 0.f;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int i = p + 4 * m;
                    if (i < r) s += sN[(16 * b + r) * T_LD + 16 * b + i] * tv[m];
                }
                s += __shfl_xor(s, 1);
                s += __shfl_xor(s, 2);
                const float tr = (r == jc ? 1.f : 0.f) - s;
                if (p == (r & 3)) tv[r >> 2] = tr;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
                sm.t[(16 * b + p + 4 * m) * T_LD + 16 * b + jc] = tv[m];
            // blocks above the diagonal are never read
        }
        __syncthreads();
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            const int b = wave;
            if (b >= d) {
                // Z = sum_{m=b-d}^{b-1} N[b][m] T[m][b-d];  T[b][b-d] = -T[b][b] Z
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                for (int m = b - d; m < b; ++m) {
                    float an[4], bt[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        an[e] = sN[(16 * b + l16) * T_LD + 16 * m + 4 * g4 + e];
                        bt[e] = sm.t[(16 * m + 4 * g4 + e) * T_LD + 16 * (b - d) + l16];
                    }
                    bf16x4 ah, al, bh, bl;
                    split4(an, ah, al);
                    split4(bt, bh, bl);
                    z = mma16x3(ah, al, bh, bl, z);
                }
                float at[4], zz[4] = {z[0], z[1], z[2], z[3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) at[e] = sm.t[(16 * b + l16) * T_LD + 16 * b + 4 * g4 + e];
                bf16x4 ah, al, bh, bl;
                split4(at, ah, al);
                split4(zz, bh, bl);
                f32x4 tr = {0.f, 0.f, 0.f, 0.f};
                tr = mma16x3(ah, al, bh, bl, tr);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.t[(16 * b + 4 * g4 + e) * T_LD + 16 * (b - d) + l16] = -tr[e];
            }
            __syncthreads();
        }

        // ================= E1: X^T = S0^T Kt^T and S0^T Qt^T (row block rb) ==
        f32x4 accO = {0.f, 0.f, 0.f, 0.f};
        {
            f32x4 accX = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int c0s = 32 * s + 8 * g4;
                const bf16x8 sh = *reinterpret_cast<const bf16x8*>(&sm.st[0][l16 * QK_LD + c0s]);
                const bf16x8 sl = *reinterpret_cast<const bf16x8*>(&sm.st[1][l16 * QK_LD + c0s]);
                float xk[8], xq[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float er = sm.erho[rb * kDim + c0s + j];
                    xk[j] = ((float)fkh[s][j] + (float)fkl[s][j]) * er;
                    xq[j] = ((float)fqh[s][j] + (float)fql[s][j]) * er;
                }
                bf16x8 kh, kl, qh, ql;
                split8(xk, kh, kl);
                split8(xq, qh, ql);
                accX = mma32x3(sh, sl, kh, kl, accX);
                accO = mma32x3(sh, sl, qh, ql, accO);
            }
            // Y^T[j][r] = beta_r (V[r][j] - X[r][j]),  j = 4 g4 + e, r = rrow
            const float br = sm.beta[rrow];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * g4 + e;
                const float yv = br * (sm.v[rrow * DVS + j] - accX[e]);
                __bf16 hi, lo;
                split1(yv, hi, lo);
                sm.y[0][j * Y_LD + rrow] = hi;
                sm.y[1][j * Y_LD + rrow] = lo;
            }
        }
        __syncthreads();

        // ================= E2: U = T Y (row block rb) ========================
        {
            f32x4 accU = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                if (ib > rb) break;
                float at[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) at[e] = sm.t[rrow * T_LD + 16 * ib + 4 * g4 + e];
                bf16x4 ah, al;
                split4(at, ah, al);
                const bf16x4 yh = *reinterpret_cast<const bf16x4*>(&sm.y[0][l16 * Y_LD + 16 * ib + 4 * g4]);
                const bf16x4 yl = *reinterpret_cast<const bf16x4*>(&sm.y[1][l16 * Y_LD + 16 * ib + 4 * g4]);
                accU = mma16x3(ah, al, yh, yl, accU);
            }
            // accU[e] = U[16rb + 4 g4 + e][l16]  ->  U^T[j = l16][r]
            float x[4] = {accU[0], accU[1], accU[2], accU[3]};
            bf16x4 hi, lo;
            split4(x, hi, lo);
            *reinterpret_cast<bf16x4*>(&sm.u[0][l16 * Y_LD + 16 * rb + 4 * g4]) = hi;
            *reinterpret_cast<bf16x4*>(&sm.u[1][l16 * Y_LD + 16 * rb + 4 * g4]) = lo;
        }
        __syncthreads();

        // ================= E3: O^T += U^T P^T; store o ========================
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            if (ib > rb) break;
            const bf16x4 uh = *reinterpret_cast<const bf16x4*>(&sm.u[0][l16 * Y_LD + 16 * ib + 4 * g4]);
            const bf16x4 ul = *reinterpret_cast<const bf16x4*>(&sm.u[1][l16 * Y_LD + 16 * ib + 4 * g4]);
            accO = mma16x3(uh, ul, pth[ib], ptl[ib], accO);
        }
        if (rrow < L) {
            // accO[e] = O^T[4 g4 + e][rrow]
            *reinterpret_cast<float4*>(o + ((row0 + c0 + rrow) * H + h) * kDim + col0 + 4 * g4) =
                make_float4(accO[0], accO[1], accO[2], accO[3]);
        }

        // ================= E4: S1 = Diag(2^G_63) S0 + Ke^T U ==================
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * wave + tt;
            const int chl = 16 * t + l16;  // channel of this lane in A-operand layout
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[tt][i] *= sm.el[16 * t + 4 * g4 + i];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int tk0 = 32 * s + 8 * g4;     // tokens tk0 .. tk0+7, one block
                const float ks = sm.kend[((tk0) >> 4) * kDim + chl];
                float x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = sm.cb[(tk0 + j) * G_LD + chl] * ks;
                bf16x8 ah, al;
                split8(x, ah, al);
                const bf16x8 uh = *reinterpret_cast<const bf16x8*>(&sm.u[0][l16 * Y_LD + tk0]);
                const bf16x8 ul = *reinterpret_cast<const bf16x8*>(&sm.u[1][l16 * Y_LD + tk0]);
                sacc[tt] = mma32x3(ah, al, uh, ul, sacc[tt]);
            }
        }
        store_state_t();
        __syncthreads();
    }

    if (final_state) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * wave + tt;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = 16 * t + 4 * g4 + i;
                final_state[unit * (kDim * kDim) + ch * kDim + col0 + l16] = sacc[tt][i];
            }
        }
    }
}

}  // namespace

hipError_t launch_prefill_chunked(const void* q, const void* k, const void* v, const void* beta,
                                  const float* log_alpha, const int32_t* cu_seqlens,
                                  int64_t n_seq, int64_t T, int64_t H,
                                  const float* initial_state, float* o, float* final_state,
                                  hipStream_t stream)
{
    const int64_t units = n_seq * H;
    if (units <= 0) return hipSuccess;
    const int64_t groups = (units + 7) / 8;
    const dim3 grid(static_cast<unsigned>(groups * 8 * NSLICE)), block(256);
    hipLaunchKernelGGL(prefill_chunked_kernel, grid, block, 0, stream,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                       static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(beta), log_alpha,
                       cu_seqlens, T, static_cast<int>(H), units, initial_state, o, final_state);
    return hipGetLastError();
}

}  // namespace kda
