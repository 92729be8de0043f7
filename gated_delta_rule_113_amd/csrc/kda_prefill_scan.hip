// Chunked KDA prefill on bf16 matrix cores with sequence segmentation.
//
// The recurrence (per head; S is d_k x d_v, rows = forgetting channels)
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t
// ("Kimi K3 -- the architecture and infrastructure, explained": section "How
// the delta rule actually works" gives the update, section "Kimi Delta
// Attention: the load-bearing choice" the per-channel gate and the blockwise,
// context-parallel organisation on matrix units) is evaluated 64 tokens at a
// time.  Within a chunk of tokens r = 0..63 entering with state S0, with G_r
// the inclusive cumulative log2-decay of each channel:
//     A_ri  = sum_c k_rc k_ic 2^(G_rc - G_ic)   (i < r)      key-key interactions
//     P_ri  = sum_c q_rc k_ic 2^(G_rc - G_ic)   (i <= r)     query-key interactions
//     T     = (I + Diag(b) A)^-1                              (UT transform)
//     X     = Kt S0,   Kt_r = k_r 2^G_r                        decayed keys
//     U     = T Diag(b) (V - X)                               corrected writes
//     O     = Qt S0 + P U,   Qt_r = q_r 2^G_r
//     S1    = Diag(2^G_63) S0 + Ke^T U,   Ke_i = k_i 2^(G_63 - G_i)
// which is the token recurrence regrouped (exact in real arithmetic).
//
// Sequence segmentation ("context parallel" within one GPU).  The chunk step
// is affine in the entering state, so a segment of the sequence maps its
// entering state to S_end = M S_start + R with M (d_k x d_k) the product of
// its chunk transitions.  A long sequence is cut into segments; pass 1 runs
// each segment but the last on the augmented state [M | R] (started from
// [I | 0]; packed input: the first segment builds R only, from the true
// initial state; dense input: the first segment instead runs with outputs,
// since its entering state is known), pass 2 composes the segment maps in
// order to get every segment's true entering state, pass 3 reruns every
// segment not yet done from its entering state and writes the outputs and the
// final state.  While pass 1 maps a chunk it also keeps the chunk's split T and
// P in a workspace, so that pass 3 loads them instead of forming them again.
// Sequences no longer than a segment take pass 3 only; those of at most 16
// tokens are left to the token-by-token kernel.
// For packed input a one-workgroup plan kernel, on the device where the
// lengths are, picks the segment length, numbers the segments (and workspace
// slots, for sequences cut in two or more) and orders them longest first.
//
// One workgroup (8 waves) processes one (sequence, head, segment); wave w
// holds value columns 16w..16w+15 of the fp32 state in matrix-core
// accumulator registers for the whole segment.  Per chunk all d_v-independent
// work (cumulative decay, A, P, the UT solve, the decayed operands) is done
// once and staged in LDS; the state products then run per wave with the state
// and the corrected writes as register operands.
//
// Precision: every matrix-core operand that is not an exact bf16 input is
// split into hi + lo bf16 parts and each product uses hi*hi + hi*lo + lo*hi
// with fp32 accumulation; the state, decay factors, T and all accumulations
// are fp32.
//
// Overflow-free decay factors: 2^(G_r - G_i) is never formed from 2^(-G_i).
// Tiles of 16 x 16 tokens pair a row factor 2^(G_r - rho) with a column factor
// 2^(rho - G_i) for a per-row-block reference rho: the block's 8th token when
// every channel's log2-decay from there to either end of the block is <= 96
// (both factors then stay within [2^-96, 2^96]), else the end of the previous
// block, in which case the diagonal tile is computed pairwise on the vector
// ALUs.  Off-diagonal column factors are always <= 1.
//
// Operand layouts.  A 16x16x32 matrix instruction sums over 32 k-slots; lane
// group g (lanes 16g..16g+15) supplies slots 8g..8g+7.  Slot (g, j) of step s
// is bound to channel (or token) 32s + 16(j >> 2) + 4g + (j & 3), so that a
// result tile in accumulator layout (lane group g holding rows 4g..4g+3) is
// directly the B operand of the next product over that index.  Tiles that are
// read as A operands are stored in LDS with the same index permutation, so
// each fragment is one 16-byte read, and XOR-swizzled by row against bank
// conflicts.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;            // tokens per chunk
constexpr int NW = 8;             // waves per workgroup
constexpr int NT = 64 * NW;       // threads per workgroup
constexpr int N_LD = CH + 4;      // fp32 row stride of 64 x 64 tiles
constexpr int SS = kDim * kDim;   // floats per state matrix
constexpr float kSafeLog2 = 96.f;
constexpr float kLog2e = 1.4426950408889634f;

// ---- LDS map (bytes).  Regions are reused within a chunk once their
//      previous contents are dead.
// R0: raw q | raw k | decay G (fp32), later the decayed operands Kt, Qt.
constexpr int OFF_Q = 0;
constexpr int OFF_K = 16384;
constexpr int OFF_G = 32768;
constexpr int R0_BYTES = 32768 + CH * kDim * 4;
constexpr int OFF_KT_HI = 0, OFF_KT_LO = 16384, OFF_QT_HI = 32768, OFF_QT_LO = 49152;
// R1: N = Diag(b) A and T (fp32) during the UT solve; later Ke^T.
constexpr int OFF_R1 = R0_BYTES;
constexpr int OFF_N = OFF_R1;
constexpr int OFF_TF = OFF_R1 + CH * N_LD * 4;
constexpr int OFF_KE_HI = OFF_R1, OFF_KE_LO = OFF_R1 + 16384;
constexpr int R1_BYTES = 2 * CH * N_LD * 4;
// T and P as split operands, the raw value tile, small vectors.
constexpr int OFF_T_HI = OFF_R1 + R1_BYTES;
constexpr int OFF_T_LO = OFF_T_HI + 8192;
constexpr int OFF_P_HI = OFF_T_LO + 8192;
constexpr int OFF_P_LO = OFF_P_HI + 8192;
// V: [token][column] bf16 rows of V_LD bytes (padded: the 16 reads of one
// lane share a base address, and the 64 lanes of a read hit distinct banks)
constexpr int V_LD = 2 * kDim + 8;
constexpr int OFF_V = OFF_P_LO + 8192;
constexpr int OFF_BETA = OFF_V + CH * V_LD;
constexpr int OFF_EL = OFF_BETA + CH * 4;
constexpr int OFF_UNSAFE = OFF_EL + kDim * 4;
// the diagonal 16x16 blocks of T (fp32, rows of TD_LD floats), apart from
// the partial sums that share phase 4 with them
constexpr int TD_LD = 20;
constexpr int OFF_TD = OFF_UNSAFE + 16 * 4;
constexpr int LDS_BYTES = OFF_TD + 4 * 16 * TD_LD * 4;
// the output tile of a chunk (64 x 128 fp32, rows of 32 float4 slots) over T
// and P, between a chunk's state products and the next chunk's staging
constexpr int OFF_OT = OFF_T_HI;
static_assert(OFF_P_LO + 8192 - OFF_T_HI == CH * kDim * 4, "output tile fits T and P exactly");
static_assert(4 * 8192 == 16 * NT * 4, "the T/P image: four 16-byte pieces per thread");
// In the workspace each of the four planes of the T/P image (T hi, T lo, P hi,
// P lo; 64 rows of eight 16-byte chunks) keeps only the chunks that can hold a
// nonzero entry: T and P are lower triangular, and logical chunk c of a row
// holds the natural columns 32 (c / 4) + 4 (c mod 4) + {0..3, 16..19}, so it is
// kept in row r when its first column 32 (c / 4) + 4 (c mod 4) <= r.  Kept
// chunks are numbered row by row: 336 per plane instead of 512.
constexpr int kTpChunks = 336;
constexpr int TP_BYTES = 4 * kTpChunks * 16;   // workspace bytes per (chunk, head)
__device__ __forceinline__ bool tp_kept(int r, int c) { return 32 * (c >> 2) + 4 * (c & 3) <= r; }
// the number of kept chunks in the rows before r
__device__ __forceinline__ int tp_row_base(int r)
{
    return r <= 4 ? r : r <= 8 ? 4 + 2 * (r - 4) : r <= 12 ? 12 + 3 * (r - 8) : r <= 32 ? 24 + 4 * (r - 12)
         : r <= 36 ? 104 + 5 * (r - 32) : r <= 40 ? 124 + 6 * (r - 36) : r <= 44 ? 148 + 7 * (r - 40)
         : 176 + 8 * (r - 44);
}
static_assert(R1_BYTES >= 32768, "Ke^T must fit in R1");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU");

// Index permutation within each group of 32 (see the header comment).
__device__ __forceinline__ int perm(int x)
{
    return (x & ~31) | ((x & 12) << 1) | ((x & 16) >> 2) | (x & 3);
}
// Byte offsets in bf16 tiles of 128 (256 B rows) and 64 (128 B rows) entries.
__device__ __forceinline__ int a256(int row, int pos)
{
    return (row << 8) + ((((pos >> 3) ^ row) & 15) << 4) + ((pos & 7) << 1);
}
__device__ __forceinline__ int a128(int row, int pos)
{
    return (row << 7) + ((((pos >> 3) ^ (row >> 1)) & 7) << 4) + ((pos & 7) << 1);
}

// Byte offset of entry `pos` (permuted channel) of token row `row` in the fp32
// decay tile: rows of 32 float4 chunks, the chunk index XOR-ed with
// (row ^ row >> 4) & 15 so that both 16 consecutive rows and 16 rows four
// apart hit distinct banks at one chunk position.
__device__ __forceinline__ int g_off(int row, int pos)
{
    return OFF_G + (row << 9) + (((((pos >> 2) ^ (row ^ (row >> 4))) & 15) | ((pos >> 2) & 16)) << 4) + ((pos & 3) << 2);
}
// Byte offset in the transposed tile Ke^T (channel rows of 64 tokens): like
// a128, with the chunk index XOR-ed with (row >> 1 ^ row >> 3) & 7, which
// keeps 16 consecutive rows conflict-free and spreads rows four apart.
__device__ __forceinline__ int ke_off(int row, int pos)
{
    return (row << 7) + ((((pos >> 3) ^ (row >> 1) ^ (row >> 3)) & 7) << 4) + ((pos & 7) << 1);
}

// byte offset of entry (row, col) of the diagonal T block b
__device__ __forceinline__ int td_off(int b, int row, int col)
{
    return OFF_TD + ((16 * b + row) * TD_LD + col) * 4;
}

// byte offset of float4 slot `slot` (0..31) of row `row` in the output tile,
// XOR-swizzled so that 16 rows written at one slot hit distinct banks
__device__ __forceinline__ int o_slot(int row, int slot)
{
    return (row << 9) + (((slot ^ row) & 31) << 4);
}

template <typename T>
__device__ __forceinline__ T& at(char* base, int off)
{
    return *reinterpret_cast<T*>(base + off);
}

// base (wave-uniform) + a 32-bit byte offset, so that the access can take the
// scalar-base + 32-bit vector-offset address form
template <typename T, typename P>
__device__ __forceinline__ T* gat(P* base, uint32_t byte_off)
{
    return reinterpret_cast<T*>(reinterpret_cast<
        typename std::conditional<std::is_const<P>::value, const char, char>::type*>(base) + byte_off);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bfw(__bf16 x) { return (float)x; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// x = hi + lo with hi = bf16(x) (round to nearest even) and lo = bf16(x - hi).
// Elements go in pairs: one packed conversion gives both hi parts, whose
// fp32 values are read back from the packed bits (a shift and a mask), so
// each element is rounded to bf16 only once for its hi part.
template <int W, typename V>
__device__ __forceinline__ void split_vec(const float (&x)[W], V& h, V& l)
{
    static_assert(W % 2 == 0 && sizeof(V) == 2 * W, "pairs of bf16");
    typedef uint32_t uv __attribute__((ext_vector_type(W / 2)));
    uv hu, lu;
#pragma unroll
    for (int j = 0; j < W; j += 2) {
        uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x[j], x[j + 1]}, bf16x2));
        asm("" : "+v"(u));  // keep the read-back on the packed bits
        const float f0 = __uint_as_float(u << 16), f1 = __uint_as_float(u & 0xffff0000u);
        hu[j / 2] = u;
        lu[j / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x[j] - f0, x[j + 1] - f1}, bf16x2));
    }
    h = __builtin_bit_cast(V, hu);
    l = __builtin_bit_cast(V, lu);
}

// hi*hi + hi*lo + lo*hi on the 16x16x32 bf16 matrix instruction.
__device__ __forceinline__ f32x4 mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
    return c;
}

// the same on the 16x16x16 instruction (used by the small UT-solve blocks)
__device__ __forceinline__ f32x4 mma16x3(bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl, f32x4 c)
{
    const i16x4 AH = __builtin_bit_cast(i16x4, ah), AL = __builtin_bit_cast(i16x4, al);
    const i16x4 BH = __builtin_bit_cast(i16x4, bh), BL = __builtin_bit_cast(i16x4, bl);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(AL, BH, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(AH, BL, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(AH, BH, c, 0, 0, 0);
    return c;
}

// x of the lane N places lower in the same 16-lane row, 0 for the first N
// lanes of each row (DPP row shift; no LDS traffic)
template <int N>
__device__ __forceinline__ float4 row_shr(float4 x)
{
    auto sh = [](float v) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + N, 0xF, 0xF, true));
    };
    return make_float4(sh(x.x), sh(x.y), sh(x.z), sh(x.w));
}

// x of lane (lane ^ M) for M = 1 or 2 (DPP quad permutation)
template <int M>
__device__ __forceinline__ float quad_xor(float x)
{
    static_assert(M == 1 || M == 2, "within a quad");
    constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false));
}

// x of the lane N places further in the same 16-lane row, cyclically (DPP row rotate)
template <int N>
__device__ __forceinline__ float row_ror(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}

// Eight consecutive bf16 entries of a token row, whose 128 entries are spread
// over the 16 lanes of one DPP row: divided by the row's L2 norm (a zero row
// stays zero) and rounded back to bf16, nearest even.
__device__ __forceinline__ uint4 unit_row(uint4 w)
{
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(u[j] << 16);
        f[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += f[j] * f[j];
    ss += row_ror<8>(ss);
    ss += row_ror<4>(ss);
    ss += row_ror<2>(ss);
    ss += row_ror<1>(ss);
    const float inv = ss > 0.f ? rsqrtf(ss) : 0.f;
    uint32_t r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        r[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){f[2 * j] * inv, f[2 * j + 1] * inv}, bf16x2));
    return make_uint4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ float4 f4add(float4 a, float4 b)
{
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

}  // namespace

// Arguments shared by the three passes (by value).
struct ScanArgs {
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    const bf16_t* beta;
    const float* log_alpha;
    const int32_t* cu_seqlens;  // packed rows, or null for dense sequences of T rows
    const int32_t* seg_first;   // packed + segmented: first segment of each sequence [n_seq + 1],
                                // then the segment length the plan chose
    const int32_t* seg_order;   // packed + segmented: segments by decreasing length (launch order)
    const int32_t* ws_first;    // packed + segmented: first workspace slot of each sequence
                                // (only sequences of two or more segments have slots)
    int64_t T;                  // dense sequence length
    int64_t n_seq;
    int64_t seg_len;            // tokens per segment (multiple of 64); 0 = one segment each
    int64_t seg0_len;           // dense: tokens of each sequence's first segment (multiple of 64)
    int seg0_out;               // dense: pass 1 runs the first segment with outputs (pass 3 skips it)
    int64_t nseg_dense;         // dense: segments per sequence
    int64_t n_segs;             // number of segment slots (grid bound)
    int H;
    StateRefs st;  // entering and leaving states (per sequence, or pool slots)
    float* o;
    int raw;       // q, k unnormalised, beta and log_alpha logits (kda.h *_raw)
    int64_t short_max;  // sequences of at most this many tokens are skipped (0: none)
    float* ws_maps;   // [slots][H][2][d_k][d_v]: M and R of each segment but the last
    float* ws_start;  // [slots][H][d_k][d_v]: entering state of each segment
    char* ws_tp;      // or null: the kept chunks (21 KiB) of the split T and P images of every chunk of the
                      // segments that pass 1 maps, for pass 3 to reuse; block (chunk id, head), with
                      // chunk id = (first row of the segment) / 64 + sequence + chunk within the segment
                      // (segments start at multiples of 64 within their sequence, so ids are unique
                      // and below rows / 64 + sequences + 1)
};

namespace {

struct SegInfo {
    int64_t n;       // sequence
    int64_t j;       // segment within the sequence
    int64_t nseg;    // segments of the sequence
    int64_t z0;      // global index of its first segment
    int64_t row0;    // first row of the sequence
    int64_t begin;   // segment rows [begin, end) relative to row0
    int64_t end;
    int64_t len;     // tokens of the whole sequence
    bool valid;
};

__device__ SegInfo decode_segment(const ScanArgs& a, int64_t z)
{
    SegInfo s;
    s.valid = z < a.n_segs;
    if (!s.valid) return s;
    int64_t len;
    if (!a.cu_seqlens) {
        s.nseg = a.nseg_dense;
        s.n = z / s.nseg;
        s.j = z - s.n * s.nseg;
        s.z0 = z - s.j;
        s.row0 = s.n * a.T;
        len = a.T;
    } else if (!a.seg_first) {
        s.n = z;
        s.j = 0;
        s.nseg = 1;
        s.z0 = z;
        s.row0 = a.cu_seqlens[z];
        len = static_cast<int64_t>(a.cu_seqlens[z + 1]) - s.row0;
    } else {
        // the sequence whose segment range holds z
        int64_t lo = 0, hi = a.n_seq;  // seg_first[lo] <= z < seg_first[hi]
        if (z >= a.seg_first[a.n_seq]) {
            s.valid = false;
            return s;
        }
        while (hi - lo > 1) {
            const int64_t mid = (lo + hi) >> 1;
            if (a.seg_first[mid] <= z) lo = mid;
            else hi = mid;
        }
        s.n = lo;
        s.z0 = a.seg_first[lo];
        s.j = z - s.z0;
        s.nseg = static_cast<int64_t>(a.seg_first[lo + 1]) - s.z0;
        s.row0 = a.cu_seqlens[lo];
        len = static_cast<int64_t>(a.cu_seqlens[lo + 1]) - s.row0;
    }
    s.len = len;
    // packed input: the segment length is the plan's choice, stored after seg_first
    const int64_t seg = s.nseg == 1 ? len : (a.seg_first ? a.seg_first[a.n_seq + 1] : a.seg_len);
    // dense: the first segment may be shorter than the others
    const int64_t seg0 = (s.nseg == 1 || a.cu_seqlens || a.seg0_len <= 0) ? seg : a.seg0_len;
    s.begin = s.j == 0 ? 0 : seg0 + (s.j - 1) * seg;
    s.end = (s.j == s.nseg - 1) ? len : (s.j == 0 ? seg0 : s.begin + seg);
    return s;
}

// One (sequence, head, segment) of a pass; sm is the workgroup's LDS.
// OUT = true : outputs and leaving state, d_v = 128 (one 16-column group per wave)
// OUT = false: segment maps [M | R], 256 columns (two groups per wave), no outputs
// With seg0_out (dense input), the first segment of a sequence cut in two or
// more runs with outputs in pass 1, from the true initial state, and leaves its
// state where pass 2 expects it; pass 3 then skips it.
// TP (with a T/P workspace): pass 1 also forms P and stores each chunk's split
// T and P; pass 3 loads them instead of forming the A and P tiles and solving
// for T (the segment's inputs are the same, so are T and P).
template <bool OUT, bool TP>
__device__ __forceinline__ void scan_segment(const ScanArgs& a, char* sm, bool pass1)
{
    constexpr int NS = OUT ? 1 : 2;
    constexpr bool LOADTP = OUT && TP;        // T and P from the workspace
    constexpr bool STORETP = !OUT && TP;      // T and P to the workspace
    constexpr bool WITHP = (OUT && !TP) || STORETP;  // the P tile is formed here
    constexpr bool QIN = OUT || STORETP;      // queries are staged

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;
    const int H = a.H;
    int64_t z = blockIdx.x / H;
    const int h = static_cast<int>(blockIdx.x - z * H);
    if (a.seg_order) {
        // packed: the longest segments first, so that short ones fill in at the end
        if (z >= a.seg_first[a.n_seq]) return;
        z = a.seg_order[z];
    }

    const SegInfo sg = decode_segment(a, z);
    if (!sg.valid) return;
    if (sg.len <= a.short_max) return;        // a short sequence: the token-by-token kernel's
    if (!OUT && sg.j == sg.nseg - 1) return;  // the last segment needs no map
    const bool first_out = a.seg0_out && sg.nseg > 1 && sg.j == 0;
    // segments that pass 1 maps, when there is a T/P workspace
    const bool tp_seg = a.ws_tp && sg.nseg > 1 && sg.j < sg.nseg - 1 && !first_out;
    if (OUT ? (first_out != pass1 || (!first_out && TP != tp_seg)) : first_out) return;
    // this segment's workspace slot (dense: the segment index; packed: the
    // sequence's first slot + j, multi-segment sequences only)
    const int64_t wz = a.ws_first ? a.ws_first[sg.n] + sg.j : z;
    const bool blkM = !OUT && sg.j > 0;       // pass 1: is the M block carried?

    const int col = 16 * wave + l16;          // this lane's value column

    // ---------------- state (accumulator layout: S[g][t][i] = row 16t+4g4+i, column col)
    f32x4 S[NS][8];
    {
        const float* init = nullptr;
        if (OUT) {
            if (sg.nseg > 1 && !first_out) init = a.ws_start + (wz * H + h) * SS;
            else init = init_state_of(a.st, sg.n, h, H);
        } else if (sg.j == 0) {
            init = init_state_of(a.st, sg.n, h, H);
        }
#pragma unroll
        for (int gi = 0; gi < NS; ++gi)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ch = 16 * t + 4 * g4 + i;
                    float x;
                    if (!OUT && gi == 0) x = (ch == col) ? 1.f : 0.f;
                    else x = init ? init[ch * kDim + col] : 0.f;
                    S[gi][t][i] = x;
                }
        if (!OUT && sg.j == 0) {
            // pass 3 starts the first segment from this copy, so that a final
            // state aliasing the initial one cannot race with it
            float* dst = a.ws_start + (wz * H + h) * SS;
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(16 * t + 4 * g4 + i) * kDim + col] = S[NS - 1][t][i];
        }
    }

    const int64_t seg_tokens = sg.end - sg.begin;
    const int64_t nch = (seg_tokens + CH - 1) / CH;
    const int64_t base = sg.row0 + sg.begin;  // first row of the segment

    // ---------------- register prefetch of one chunk of inputs
    uint4 pq[2], pk[2], pv[2];
    float4 pla[4];
    bf16_t pb = {0};  // raw bits: widened when staged, so no wait follows the load
    // Addresses: a wave-uniform 64-bit pointer to the chunk's first row plus a
    // 32-bit per-lane element offset (rows of one chunk lie within
    // 64 * H * 128 elements, H <= 65536).
    const uint32_t rs = static_cast<uint32_t>(H) * kDim;  // elements per row
    // part 0 / 1: q, k, v rows (tid >> 4) + 32 part, columns 8 (tid & 15) .. +7;
    // part 2 / 3: log_alpha of token groups 2 (part - 2) .. +1 (wave w takes
    // channels 16w..16w+15; lane = token group tg = lane & 15: rows 4tg..4tg+3,
    // channel quad lane >> 4), and with part 3 beta.  The four parts are
    // issued at different points so that the vector memory requests do not
    // queue up at once.  Rows from L on read as zeros.
    auto prefetch = [&](int64_t c0, int L, int tid, int part) {
        const int64_t e0 = ((base + c0) * H + h) * kDim;
        if (part < 2) {
            const int m = part;
            const uint32_t off = __umul24(static_cast<uint32_t>(tid >> 4), rs) + 8 * (tid & 15) + m * 32 * rs;
            if (L == CH || (tid >> 4) + 32 * m < L) {
                pk[m] = *gat<const uint4>(a.k + e0, 2 * off);
                pv[m] = *gat<const uint4>(a.v + e0, 2 * off);
                if (QIN) pq[m] = *gat<const uint4>(a.q + e0, 2 * off);
            } else {
                pk[m] = pv[m] = pq[m] = make_uint4(0, 0, 0, 0);
            }
        } else {
            const uint32_t o2 = __umul24(static_cast<uint32_t>(4 * (tid & 15)), rs) + 16 * (tid >> 6) +
                                4 * ((tid & 63) >> 4);
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
                const int m = 2 * (part - 2) + mm;
                pla[m] = (L == CH || 4 * (tid & 15) + m < L)
                             ? *gat<const float4>(a.log_alpha + e0, 4 * (o2 + m * rs))
                             : make_float4(0.f, 0.f, 0.f, 0.f);
            }
            if (part == 3 && tid < CH)
                pb = tid < L ? *gat<const bf16_t>(a.beta + ((base + c0) * H + h),
                                                  2 * __umul24(static_cast<uint32_t>(tid), H))
                             : bf16_t{0};
        }
    };
    if (nch > 0)
        for (int part = 0; part < 4; ++part) prefetch(0, static_cast<int>(std::min<int64_t>(CH, seg_tokens)), tid, part);

    // whole rows of the output tile of the chunk at c0 (L rows) from LDS to o;
    // thread t covers float4 slots t + 512 j: rows (t >> 5) + 16 j
    auto store_o = [&](int64_t cp, int L, int tid) {
        float* oc = a.o + ((base + cp) * H + h) * kDim;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = (tid >> 5) + 16 * j, slot = tid & 31;
            if (row < L)
                *gat<f32x4>(oc, 4 * (__umul24(static_cast<uint32_t>(row), rs) + 4 * slot)) =
                    at<f32x4>(sm, OFF_OT + o_slot(row, slot));
        }
    };

    for (int64_t ci = 0; ci < nch; ++ci) {
        const int64_t c0 = ci * CH;
        const int L = static_cast<int>(std::min<int64_t>(CH, seg_tokens - c0));
        // Lane-derived offsets are recomputed every chunk from an opaque copy of
        // the thread index: hoisted out of the loop they would each hold a
        // register for the whole segment.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        const int l16 = lane & 15;
        const int g4 = lane >> 4;
        const int col = 16 * wave + l16;
        const int tq = tid >> 5;                 // token quad (scan, operand formation)
        const int cq = tid & 31;                 // natural channel quad
        const int pq4 = perm(4 * cq);            // its position in the permuted order
        // this chunk's T/P image in the workspace: 512 threads x 4 x 16 bytes
        char* tpg = TP ? a.ws_tp + (((sg.row0 + sg.begin) / CH + sg.n + ci) * H + h) * static_cast<int64_t>(TP_BYTES)
                       : nullptr;
        uint4 tp0, tp1, tp2, tp3;  // (named registers: an array here ended up in scratch memory)
        // this thread's 16-byte chunk of each image plane: row tid / 8, slot tid
        // mod 8, logical chunk slot ^ (row / 2 mod 8) (the a128 swizzle); a
        // chunk not kept reads chunk 0 and is replaced by zeros when staged
        const int tp_r = tid >> 3, tp_c = (tid & 7) ^ ((tp_r >> 1) & 7);
        const bool tp_in = tp_kept(tp_r, tp_c);
        if (LOADTP) {
            const uint32_t ci = tp_in ? tp_row_base(tp_r) + tp_c : 0;
            tp0 = *gat<const uint4>(tpg, 16 * ci);
            tp1 = *gat<const uint4>(tpg, 16 * (ci + kTpChunks));
            tp2 = *gat<const uint4>(tpg, 16 * (ci + 2 * kTpChunks));
            tp3 = *gat<const uint4>(tpg, 16 * (ci + 3 * kTpChunks));
        }

        // ======== 0: stage the chunk; scan of the log2-decay in registers.
        //             With outputs, the previous chunk's output tile is then
        //             written out from LDS (after the staging, whose waits for
        //             the prefetched inputs then need not count the stores or
        //             wait for the T/P loads issued after the prefetch).
        {
            if (a.raw) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    pk[m] = unit_row(pk[m]);
                    if (QIN) pq[m] = unit_row(pq[m]);
                }
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int r = (tid >> 4) + 32 * m;
                const int c8 = 8 * (tid & 15);
                const int p0 = perm(c8), p1 = perm(c8 + 4);
                at<uint2>(sm, OFF_K + a256(r, p0)) = make_uint2(pk[m].x, pk[m].y);
                at<uint2>(sm, OFF_K + a256(r, p1)) = make_uint2(pk[m].z, pk[m].w);
                if (QIN) {
                    at<uint2>(sm, OFF_Q + a256(r, p0)) = make_uint2(pq[m].x, pq[m].y);
                    at<uint2>(sm, OFF_Q + a256(r, p1)) = make_uint2(pq[m].z, pq[m].w);
                }
                at<uint2>(sm, OFF_V + r * V_LD + 2 * c8) = make_uint2(pv[m].x, pv[m].y);
                at<uint2>(sm, OFF_V + r * V_LD + 2 * c8 + 8) = make_uint2(pv[m].z, pv[m].w);
            }
            if (tid < CH)
                at<float>(sm, OFF_BETA + 4 * tid) =
                    !a.raw ? widen(pb) : (tid < L ? sigmoid_gate(widen(pb)) : 0.f);
            // this lane: channels 16*wave + 4*(lane >> 4) .. +3, tokens 4*tg .. 4*tg+3
            // with tg = lane & 15, so the 16 token groups of a channel quad
            // are one 16-lane row and the scan over them stays within the row
            const int tg = lane & 15;
            const int chn = 16 * wave + 4 * (lane >> 4);
            float4 gp[4];
            float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 x = pla[m];
                if (a.raw) {
                    // gate logits; rows past the chunk's end keep a zero log-decay
                    // (formed for every row, then selected: no branch)
                    const float4 ga = make_float4(log2_alpha_from_logit(x.x), log2_alpha_from_logit(x.y),
                                                  log2_alpha_from_logit(x.z), log2_alpha_from_logit(x.w));
                    const bool in = 4 * tg + m < L;
                    run = make_float4(run.x + (in ? ga.x : 0.f), run.y + (in ? ga.y : 0.f),
                                      run.z + (in ? ga.z : 0.f), run.w + (in ? ga.w : 0.f));
                } else {
                    run = make_float4(run.x + x.x * kLog2e, run.y + x.y * kLog2e, run.z + x.z * kLog2e,
                                      run.w + x.w * kLog2e);
                }
                gp[m] = run;
            }
            // inclusive scan of the 4-token sums over the 16 token groups
            float4 inc = run;
            inc = f4add(inc, row_shr<1>(inc));
            inc = f4add(inc, row_shr<2>(inc));
            inc = f4add(inc, row_shr<4>(inc));
            inc = f4add(inc, row_shr<8>(inc));
            const float4 exc = make_float4(inc.x - run.x, inc.y - run.y, inc.z - run.z, inc.w - run.w);
            const int pc = perm(chn);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                at<float4>(sm, g_off(4 * tg + m, pc)) = f4add(gp[m], exc);
            if (tg == 15)
                at<float4>(sm, OFF_EL + 4 * chn) =
                    make_float4(ex2(inc.x), ex2(inc.y), ex2(inc.z), ex2(inc.w));
            // Per row block rb, is the mid-block reference safe for every channel?
            // inc is G at token 4tg+3; the lane with tg = 4rb+3 compares G at tokens
            // 16rb-1 (zero for rb = 0), 16rb+7 and 16rb+15.
            const float4 gm = row_shr<2>(inc);
            const float4 gs = row_shr<4>(inc);
            const bool bad = (tg & 3) == 3 &&
                             (gs.x - gm.x > kSafeLog2 || gm.x - inc.x > kSafeLog2 ||
                              gs.y - gm.y > kSafeLog2 || gm.y - inc.y > kSafeLog2 ||
                              gs.z - gm.z > kSafeLog2 || gm.z - inc.z > kSafeLog2 ||
                              gs.w - gm.w > kSafeLog2 || gm.w - inc.w > kSafeLog2);
            const uint64_t bm = __ballot(bad);
            int flags = 0;
#pragma unroll
            for (int rbi = 0; rbi < 4; ++rbi)
                if (bm & (0x0001000100010001ull << (4 * rbi + 3))) flags |= 1 << rbi;
            if (lane == 0) at<int>(sm, OFF_UNSAFE + 4 * wave) = flags;
        }
        if (OUT && ci > 0) store_o(c0 - CH, CH, tid);
        __syncthreads();

        // ======== 3: A and P tiles.  Wave (rb, kh) covers row block rb over the
        //             channel half kh; the two halves are summed in phase 4.
        const int kh = wave >> 2;
        const int rb = kh ? 3 - (wave & 3) : (wave & 3);
        f32x4 accA[4], accP[4];
        float qk = 0.f;
        if constexpr (!LOADTP) {
            // Row blocks 2 and 3 have the most tiles; each shares its SIMD with
            // the wave of row block 1 or 0, which then issues in their gaps
            // (2% faster per call than equal priority, timed alternately).
            if (rb >= 2) __builtin_amdgcn_s_setprio(1);
            int fl = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) fl |= at<int>(sm, OFF_UNSAFE + 4 * w);
            const bool uns = (fl >> rb) & 1;
            const int r = 16 * rb + l16;  // this lane's token in row-operand position
            bf16x8 fkh[2], fkl[2], fqh[2], fql[2], cdh[2], cdl[2];
            float rho[2][8];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                const int p0 = 32 * (2 * kh + sl) + 8 * g4;
                const float4 ga = at<float4>(sm, g_off(r, p0));
                const float4 gb = at<float4>(sm, g_off(r, p0 + 4));
                float4 ra, rbv;
                if (!uns) {
                    ra = at<float4>(sm, g_off(16 * rb + 7, p0));
                    rbv = at<float4>(sm, g_off(16 * rb + 7, p0 + 4));
                } else if (rb > 0) {
                    ra = at<float4>(sm, g_off(16 * rb - 1, p0));
                    rbv = at<float4>(sm, g_off(16 * rb - 1, p0 + 4));
                } else {
                    ra = rbv = make_float4(0.f, 0.f, 0.f, 0.f);
                }
                const float gr[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
                const float rr[8] = {ra.x, ra.y, ra.z, ra.w, rbv.x, rbv.y, rbv.z, rbv.w};
                const bf16x8 kk = at<bf16x8>(sm, OFF_K + a256(r, p0));
                bf16x8 qq = kk;
                if (WITHP) qq = at<bf16x8>(sm, OFF_Q + a256(r, p0));
                float xk[8], xq[8], xd[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    rho[sl][jj] = rr[jj];
                    const float d = gr[jj] - rr[jj];
                    const float f = ex2(d);
                    xk[jj] = bfw(kk[jj]) * f;
                    xq[jj] = bfw(qq[jj]) * f;
                    xd[jj] = uns ? 0.f : bfw(kk[jj]) * ex2(-d);
                }
                split_vec(xk, fkh[sl], fkl[sl]);
                if (WITHP) split_vec(xq, fqh[sl], fql[sl]);
                split_vec(xd, cdh[sl], cdl[sl]);
            }
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                accA[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
                accP[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (ib > rb) continue;
                if (ib == rb) {
                    if (!uns) {
#pragma unroll
                        for (int sl = 0; sl < 2; ++sl) {
                            accA[ib] = mma3(cdh[sl], cdl[sl], fkh[sl], fkl[sl], accA[ib]);
                            if (WITHP) accP[ib] = mma3(cdh[sl], cdl[sl], fqh[sl], fql[sl], accP[ib]);
                        }
                    } else {
                        // steep decay inside the block: pairwise on the vector ALUs,
                        // result in the accumulator layout (row r, column 16rb+4g4+i)
                        const char* K = sm + OFF_K;
                        const char* Q = sm + (WITHP ? OFF_Q : OFF_K);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int ti = 16 * rb + 4 * g4 + i;
                            float sa = 0.f, sp = 0.f;
                            if (ti <= r) {
                                for (int p = 64 * kh; p < 64 * kh + 64; ++p) {
                                    const float f = ex2(at<float>(sm, g_off(r, p)) - at<float>(sm, g_off(ti, p)));
                                    const float ki = bfw(*reinterpret_cast<const __bf16*>(K + a256(ti, p)));
                                    const float kr = bfw(*reinterpret_cast<const __bf16*>(K + a256(r, p)));
                                    const float qr = bfw(*reinterpret_cast<const __bf16*>(Q + a256(r, p)));
                                    sa += kr * ki * f;
                                    sp += qr * ki * f;
                                }
                            }
                            accA[ib][i] = sa;
                            accP[ib][i] = sp;
                        }
                    }
                } else {
                    const int ti = 16 * ib + l16;  // this lane's token in column position
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl) {
                        const int p0 = 32 * (2 * kh + sl) + 8 * g4;
                        const float4 ga = at<float4>(sm, g_off(ti, p0));
                        const float4 gb = at<float4>(sm, g_off(ti, p0 + 4));
                        const float gi[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
                        const bf16x8 kk = at<bf16x8>(sm, OFF_K + a256(ti, p0));
                        float x[8];
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj) x[jj] = bfw(kk[jj]) * ex2(rho[sl][jj] - gi[jj]);
                        bf16x8 ch, cl;
                        split_vec(x, ch, cl);
                        accA[ib] = mma3(ch, cl, fkh[sl], fkl[sl], accA[ib]);
                        if (WITHP) accP[ib] = mma3(ch, cl, fqh[sl], fql[sl], accP[ib]);
                    }
                }
            }
            // P_rr = q_r . k_r carries no decay; it is summed in fp32 here, since
            // when it dominates o_r (a token right after a zero state) its
            // cancellation would expose the ~16-bit split operands
            if (WITHP && kh == 1) {
#pragma unroll
                for (int part = 0; part < 4; ++part) {
                    const int p0 = 32 * g4 + 8 * part;
                    const bf16x8 kk = at<bf16x8>(sm, OFF_K + a256(r, p0));
                    const bf16x8 qq = at<bf16x8>(sm, OFF_Q + a256(r, p0));
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) qk += bfw(qq[jj]) * bfw(kk[jj]);
                }
                qk += __shfl_xor(qk, 16);
                qk += __shfl_xor(qk, 32);
            }
            // accA[ib][i] = A[r][16ib+4g4+i] and accP likewise, over this
            // channel half.  The halves are summed in phase 4 by the waves that
            // finish each product: the second half parks its A, the first its P.
            if (kh == 1) {
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    if (ib > rb) continue;
                    at<f32x4>(sm, OFF_N + (r * N_LD + 16 * ib + 4 * g4) * 4) = accA[ib];
                }
            } else if (WITHP) {
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    if (ib > rb) continue;
                    at<f32x4>(sm, OFF_TF + (r * N_LD + 16 * ib + 4 * g4) * 4) = accP[ib];
                }
            }
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
        }

        // ======== 4: the first half of the waves (row block rb = wave) finishes
        //             N = Diag(b) A (strictly lower) of its row block and, from
        //             it, the diagonal block T[rb][rb] = (I + N[rb][rb])^-1 by
        //             forward substitution; the second half finishes P (lower,
        //             split) of its row block.  Then every thread forms its share
        //             of the decayed operands.
        // Operand formation: thread (tq, cq) covers tokens
        // 4tq..4tq+3 x channels 4cq..4cq+3 of Kt, Qt and Ke, held in registers
        // until their LDS regions are free.
        bf16x4 fKh[4], fKl[4], fQh[4], fQl[4], fEh[4], fEl[4];
        auto form = [&]() {
            const float4 g63 = at<float4>(sm, g_off(63, pq4));
            float ke[4][4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 4 * tq + m;
                const float4 gv = at<float4>(sm, g_off(r, pq4));
                const bf16x4 kv = at<bf16x4>(sm, OFF_K + a256(r, pq4));
                bf16x4 qv = kv;
                if (OUT) qv = at<bf16x4>(sm, OFF_Q + a256(r, pq4));
                const float g[4] = {gv.x, gv.y, gv.z, gv.w};
                const float e63[4] = {g63.x, g63.y, g63.z, g63.w};
                float xk[4], xq[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float e = ex2(g[x]);
                    xk[x] = bfw(kv[x]) * e;
                    xq[x] = bfw(qv[x]) * e;
                    ke[x][m] = bfw(kv[x]) * ex2(e63[x] - g[x]);
                }
                split_vec(xk, fKh[m], fKl[m]);
                if (OUT) split_vec(xq, fQh[m], fQl[m]);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) split_vec(ke[x], fEh[x], fEl[x]);
        };
        // T is consumed as a split A operand: [token][token] bf16 hi and lo,
        // column index permuted like every other k-slot index.
        auto put_t = [&](int row, int tok, float x) {
            const __bf16 hb = (__bf16)x;
            const int off = a128(row, perm(tok));
            at<__bf16>(sm, OFF_T_HI + off) = hb;
            at<__bf16>(sm, OFF_T_LO + off) = (__bf16)(x - (float)hb);
        };

        if constexpr (LOADTP) {
            // the output tile over T and P was written out in phase 0.  A chunk
            // not kept is overwritten with zeros after its (dummy) copy: a select
            // on the loaded value would be compiled to wait for the load at once
            at<uint4>(sm, OFF_T_HI + 16 * tid) = tp0;
            at<uint4>(sm, OFF_T_HI + 16 * (tid + NT)) = tp1;
            at<uint4>(sm, OFF_T_HI + 16 * (tid + 2 * NT)) = tp2;
            at<uint4>(sm, OFF_T_HI + 16 * (tid + 3 * NT)) = tp3;
            if (!tp_in) {
                const uint4 z4 = make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j) at<uint4>(sm, OFF_T_HI + 16 * (tid + NT * j)) = z4;
            }
        } else if (kh == 0) {
            const int r = 16 * rb + l16;
            const float br = at<float>(sm, OFF_BETA + 4 * r);
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                if (ib > rb) continue;
                const int o4 = (r * N_LD + 16 * ib + 4 * g4) * 4;
                const f32x4 pa = at<f32x4>(sm, OFF_N + o4);
                f32x4 nn;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ti = 16 * ib + 4 * g4 + i;
                    nn[i] = ti < r ? br * (pa[i] + accA[ib][i]) : 0.f;
                }
                at<f32x4>(sm, OFF_N + o4) = nn;
            }
            // T[b][b] for b = rb from this wave's own diagonal N block (read
            // back in order after its writes); lane (jc, p) holds rows
            // 4p..4p+3 of column jc
            const int b = rb, jc = lane >> 2, p = lane & 3;
            float4 nv[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
                nv[rr] = at<float4>(sm, OFF_N + ((16 * b + rr) * N_LD + 16 * b + 4 * p) * 4);
            float tv[4] = {0.f, 0.f, 0.f, 0.f};  // T[16b + 4p + m][16b + jc]
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                // N is strictly lower, so entries at or right of the diagonal are zero
                float s = nv[rr].x * tv[0] + nv[rr].y * tv[1] + nv[rr].z * tv[2] + nv[rr].w * tv[3];
                s += quad_xor<1>(s);
                s += quad_xor<2>(s);
                const float tr = (rr == jc ? 1.f : 0.f) - s;
                if (p == (rr >> 2)) tv[rr & 3] = tr;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                at<float>(sm, td_off(b, 4 * p + m, jc)) = tv[m];
                put_t(16 * b + 4 * p + m, 16 * b + jc, tv[m]);
            }
        } else if (WITHP) {
            const int r = 16 * rb + l16;
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                if (ib <= rb) {
                    const f32x4 pp = at<f32x4>(sm, OFF_TF + (r * N_LD + 16 * ib + 4 * g4) * 4);
                    float x[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int ti = 16 * ib + 4 * g4 + i;
                        x[i] = ti < r ? pp[i] + accP[ib][i] : (ti == r ? qk : 0.f);
                    }
                    bf16x4 hi, lo;
                    split_vec(x, hi, lo);
                    const int pp0 = perm(16 * ib + 4 * g4);
                    at<bf16x4>(sm, OFF_P_HI + a128(r, pp0)) = hi;
                    at<bf16x4>(sm, OFF_P_LO + a128(r, pp0)) = lo;
                } else if (ib == rb + 1 && (rb & 1) == 0) {
                    // the upper tile that shares a 32-token step with the diagonal
                    const int pp0 = perm(16 * ib + 4 * g4);
                    const bf16x4 zz = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
                    at<bf16x4>(sm, OFF_P_HI + a128(r, pp0)) = zz;
                    at<bf16x4>(sm, OFF_P_LO + a128(r, pp0)) = zz;
                }
            }
        }
        form();
        __syncthreads();

        // ======== 6: off-diagonal blocks by block column a (wave a, no barrier):
        //             T[b][a] = -T[b][b] sum_{m=a}^{b-1} N[b][m] T[m][a].  The
        //             blocks of one column stay in this wave's registers, in
        //             accumulator layout, which is the B layout of the next
        //             16x16x16 product.  Meanwhile the other waves store Kt, Qt
        //             (q, k and G are dead) and the zero upper tiles that share
        //             a 32-token step with a diagonal tile.
        {
            auto column = [&](auto ac) {
                constexpr int A = decltype(ac)::value;
                // every N and diagonal-T block of this column's chain, read up front
                float4 nb[4][4], db[4];
#pragma unroll
                for (int b = A + 1; b < 4; ++b) {
#pragma unroll
                    for (int m = A; m < b; ++m)
                        nb[b][m] = at<float4>(sm, OFF_N + ((16 * b + l16) * N_LD + 16 * m + 4 * g4) * 4);
                    db[b] = at<float4>(sm, td_off(b, l16, 4 * g4));
                }
                bf16x4 bh[4], bl[4];
                {
                    float da[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        da[e] = at<float>(sm, td_off(A, 4 * g4 + e, l16));
                    split_vec(da, bh[A], bl[A]);
                }
#pragma unroll
                for (int b = A + 1; b < 4; ++b) {
                    f32x4 zacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = A; m < b; ++m) {
                        const float4 n4 = nb[b][m];
                        const float an[4] = {n4.x, n4.y, n4.z, n4.w};
                        bf16x4 ah, al;
                        split_vec(an, ah, al);
                        zacc = mma16x3(ah, al, bh[m], bl[m], zacc);
                    }
                    const float4 d4 = db[b];
                    const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
                    const float zz[4] = {zacc[0], zacc[1], zacc[2], zacc[3]};
                    bf16x4 ah, al, zh, zl;
                    split_vec(dd, ah, al);
                    split_vec(zz, zh, zl);
                    f32x4 tr = {0.f, 0.f, 0.f, 0.f};
                    tr = mma16x3(ah, al, zh, zl, tr);
                    const float tb[4] = {-tr[0], -tr[1], -tr[2], -tr[3]};
                    split_vec(tb, bh[b], bl[b]);
                    // tb[e] = T[16b + 4g4 + e][16A + l16]
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int off = a128(16 * b + 4 * g4 + e, perm(16 * A + l16));
                        at<__bf16>(sm, OFF_T_HI + off) = bh[b][e];
                        at<__bf16>(sm, OFF_T_LO + off) = bl[b][e];
                    }
                }
            };
            if (LOADTP) {
            } else if (wave == 0) column(std::integral_constant<int, 0>{});
            else if (wave == 1) column(std::integral_constant<int, 1>{});
            else if (wave == 2) column(std::integral_constant<int, 2>{});
            else if (wave == 3 || wave == 4) {
                // tile (0,1) or (2,3): rows 16rb.., tokens 16rb+16..; lane = (row, 4-token group)
                const int rb0 = wave == 3 ? 0 : 2;
                const int r = 16 * rb0 + (lane >> 2);
                const int pz = perm(16 * rb0 + 16 + 4 * (lane & 3));
                const bf16x4 zz = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
                at<bf16x4>(sm, OFF_T_HI + a128(r, pz)) = zz;
                at<bf16x4>(sm, OFF_T_LO + a128(r, pz)) = zz;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int rr = 4 * tq + m;
                at<bf16x4>(sm, OFF_KT_HI + a256(rr, pq4)) = fKh[m];
                at<bf16x4>(sm, OFF_KT_LO + a256(rr, pq4)) = fKl[m];
                if (OUT) {
                    at<bf16x4>(sm, OFF_QT_HI + a256(rr, pq4)) = fQh[m];
                    at<bf16x4>(sm, OFF_QT_LO + a256(rr, pq4)) = fQl[m];
                }
            }
        }
        __syncthreads();

        // ======== 8: state products (each wave its own columns)
        // Ke^T into R1 (N and T are dead); read only after the next barrier
        {
            const int tp = perm(4 * tq);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                at<bf16x4>(sm, OFF_KE_HI + ke_off(4 * cq + x, tp)) = fEh[x];
                at<bf16x4>(sm, OFF_KE_LO + ke_off(4 * cq + x, tp)) = fEl[x];
            }
        }
        bf16x8 uh[NS][2], ul[NS][2];
        f32x4 O[4];
        {
            f32x4 X[NS][4];
#pragma unroll
            for (int gi = 0; gi < NS; ++gi)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) X[gi][q4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) O[q4] = f32x4{0.f, 0.f, 0.f, 0.f};
            // X = Kt S, then O = Qt S (two passes keep fewer fragments live).
            // The A fragments of step s+1 are requested before the products of
            // step s; the scheduling barriers keep the compiler from sinking
            // those reads back next to their use.
            // The state is split once per chunk; the fragment of step s+1 is
            // split while the products of step s run.
            bf16x8 shs[NS][4], sls[NS][4];
            auto split_s = [&](int s) {
#pragma unroll
                for (int gi = 0; gi < NS; ++gi) {
                    float x[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) x[jj] = S[gi][2 * s + (jj >> 2)][jj & 3];
                    split_vec(x, shs[gi][s], sls[gi][s]);
                }
            };
            split_s(0);
            // Y = Diag(b) (V - X) for the four tokens 16 q4 + 4 g4 .. +3 of this
            // lane.  With outputs it is formed during the O pass, one row block
            // per step, so that its vector work overlaps the matrix products.
            float y[NS][4][4];
            auto make_y = [&](int q4) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tk = 16 * q4 + 4 * g4 + i;
                    const float bt = at<float>(sm, OFF_BETA + 4 * tk);
                    const float vv = bfw(at<__bf16>(sm, OFF_V + tk * V_LD + 2 * col));
#pragma unroll
                    for (int gi = 0; gi < NS; ++gi) {
                        const bool zero_v = (NS == 2 && gi == 0);  // the M block has no writes
                        y[gi][q4][i] = bt * ((zero_v ? 0.f : vv) - X[gi][q4][i]);
                    }
                }
            };
#pragma unroll
            for (int pass = 0; pass < (OUT ? 2 : 1); ++pass) {
                const int oh = pass == 0 ? OFF_KT_HI : OFF_QT_HI;
                const int ol = pass == 0 ? OFF_KT_LO : OFF_QT_LO;
                bf16x8 fh[2][4], fl[2][4];
                auto fetch = [&](int s, int buf) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int off = a256(16 * q4 + l16, 32 * s + 8 * g4);
                        fh[buf][q4] = at<bf16x8>(sm, oh + off);
                        fl[buf][q4] = at<bf16x8>(sm, ol + off);
                    }
                };
                fetch(0, 0);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (s + 1 < 4) fetch(s + 1, (s + 1) & 1);
                    __builtin_amdgcn_sched_barrier(0);
                    bf16x8 sh[NS], sl[NS];
#pragma unroll
                    for (int gi = 0; gi < NS; ++gi) {
                        sh[gi] = shs[gi][s];
                        sl[gi] = sls[gi][s];
                    }
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        if (pass == 0) {
#pragma unroll
                            for (int gi = 0; gi < NS; ++gi) {
                                if (NS == 2 && gi == 0 && !blkM) continue;
                                X[gi][q4] = mma3(fh[s & 1][q4], fl[s & 1][q4], sh[gi], sl[gi], X[gi][q4]);
                            }
                        } else {
                            // O^T = S^T Qt^T: the split state fragment is the A operand
                            // and the Qt fragment the B operand, so each lane ends up
                            // with four adjacent output columns of one token
                            O[q4] = mma3(sh[0], sl[0], fh[s & 1][q4], fl[s & 1][q4], O[q4]);
                        }
                    }
                    if (pass == 0 && s + 1 < 4) split_s(s + 1);
                    if (pass == 0 && ci + 1 < nch) {
                        // a quarter of the next chunk's inputs, in flight during the
                        // rest of this one
                        const int64_t c1 = c0 + CH;
                        prefetch(c1, static_cast<int>(std::min<int64_t>(CH, seg_tokens - c1)), tid, s);
                    }
                    if (pass == 1) make_y(s);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (STORETP) {
                // T and P are complete and only read from here on: their image
                // goes to the workspace for pass 3 (here, after the X pass,
                // rather than before it: 2% per call)
                if (tp_in) {
                    const uint32_t ci = tp_row_base(tp_r) + tp_c;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *gat<uint4>(tpg, 16 * (ci + kTpChunks * j)) = at<uint4>(sm, OFF_T_HI + 16 * (tid + NT * j));
                }
            }
            if (!OUT) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) make_y(q4);
            }
            // T fragments for U = T Y, requested before the vector work on Y
            bf16x8 tfh[6], tfl[6];  // (q4, s) pairs with s <= q4/2, in order
            {
                int n = 0;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                    for (int s = 0; s <= (q4 >> 1); ++s) {
                        const int off = a128(16 * q4 + l16, 32 * s + 8 * g4);
                        tfh[n] = at<bf16x8>(sm, OFF_T_HI + off);
                        tfl[n] = at<bf16x8>(sm, OFF_T_LO + off);
                        ++n;
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
            // Y split as B operands over tokens
            bf16x8 yh[NS][2], yl[NS][2];
            {
#pragma unroll
                for (int gi = 0; gi < NS; ++gi)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        float x[8];
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj) x[jj] = y[gi][2 * s + (jj >> 2)][jj & 3];
                        split_vec(x, yh[gi][s], yl[gi][s]);
                    }
            }
            // U = T Y (T is block lower triangular: row block q4 needs steps s <= q4/2)
            f32x4 U[NS][4];
            {
                int n = 0;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
                    for (int gi = 0; gi < NS; ++gi) U[gi][q4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s <= (q4 >> 1); ++s) {
#pragma unroll
                        for (int gi = 0; gi < NS; ++gi) {
                            if (NS == 2 && gi == 0 && !blkM) continue;
                            U[gi][q4] = mma3(tfh[n], tfl[n], yh[gi][s], yl[gi][s], U[gi][q4]);
                        }
                        ++n;
                    }
                }
            }
            // P fragments for O += P U, requested before the vector work on U
            bf16x8 pfh[6], pfl[6];
            if (OUT) {
                int n = 0;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                    for (int s = 0; s <= (q4 >> 1); ++s) {
                        const int off = a128(16 * q4 + l16, 32 * s + 8 * g4);
                        pfh[n] = at<bf16x8>(sm, OFF_P_HI + off);
                        pfl[n] = at<bf16x8>(sm, OFF_P_LO + off);
                        ++n;
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int gi = 0; gi < NS; ++gi)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    float x[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) x[jj] = U[gi][2 * s + (jj >> 2)][jj & 3];
                    split_vec(x, uh[gi][s], ul[gi][s]);
                }
            if (OUT) {
                // O^T += U^T P^T (U's split fragments as A, P's as B):
                // O[q4][i] = o[token 16 q4 + l16][column 16 wave + 4 g4 + i]
                int n = 0;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
                    for (int s = 0; s <= (q4 >> 1); ++s) {
                        O[q4] = mma3(uh[0][s], ul[0][s], pfh[n], pfl[n], O[q4]);
                        ++n;
                    }
                }
            }
        }
        __syncthreads();

        // ======== 9: S <- Diag(2^G_63) S + Ke^T U (fragments of tile t+1 in
        //             flight during the products of tile t).  With outputs,
        //             the chunk's output tile first goes to LDS (over T and P,
        //             now dead); it is written out by whole rows while the next
        //             chunk is staged.  A wave's own 16 columns span 16 rows per
        //             store instruction; whole rows span 2.
        if (OUT) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int row = 16 * q4 + l16;
                at<f32x4>(sm, OFF_OT + o_slot(row, 4 * wave + g4)) = O[q4];
            }
        }
        {
            bf16x8 eh[2][2], el[2][2];
            auto fetch = [&](int t, int buf) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int off = ke_off(16 * t + l16, 32 * s + 8 * g4);
                    eh[buf][s] = at<bf16x8>(sm, OFF_KE_HI + off);
                    el[buf][s] = at<bf16x8>(sm, OFF_KE_LO + off);
                }
            };
            fetch(0, 0);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (t + 1 < 8) fetch(t + 1, (t + 1) & 1);
                const float4 e4 = at<float4>(sm, OFF_EL + (16 * t + 4 * g4) * 4);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int gi = 0; gi < NS; ++gi) {
                    S[gi][t][0] *= e4.x;
                    S[gi][t][1] *= e4.y;
                    S[gi][t][2] *= e4.z;
                    S[gi][t][3] *= e4.w;
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
#pragma unroll
                    for (int gi = 0; gi < NS; ++gi) {
                        if (NS == 2 && gi == 0 && !blkM) continue;
                        S[gi][t] = mma3(eh[t & 1][s], el[t & 1][s], uh[gi][s], ul[gi][s], S[gi][t]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();
    }

    // ---------------- results
    if (OUT && nch > 0) {
        const int64_t cl = (nch - 1) * CH;
        store_o(cl, static_cast<int>(seg_tokens - cl), tid);
    }
    if (OUT) {
        float* dst = first_out ? a.ws_start + ((wz + 1) * H + h) * SS
                               : (sg.j == sg.nseg - 1 ? final_state_of(a.st, sg.n, h, H) : nullptr);
        if (dst) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(16 * t + 4 * g4 + i) * kDim + col] = S[0][t][i];
        }
    } else if (sg.j == 0) {
        float* dst = a.ws_start + ((wz + 1) * H + h) * SS;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(16 * t + 4 * g4 + i) * kDim + col] = S[NS - 1][t][i];
    } else {
        float* dm = a.ws_maps + ((wz * H + h) * 2) * SS;
#pragma unroll
        for (int gi = 0; gi < NS; ++gi)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dm[gi * SS + (16 * t + 4 * g4 + i) * kDim + col] = S[gi][t][i];
    }
}

// PASS3 = false: pass 1 (segment maps; with seg0_out also the first segments'
// outputs); PASS3 = true: pass 3 (outputs and final states).
// TP: with the T/P workspace (a.ws_tp set).
template <bool PASS3, bool TP>
__global__ __launch_bounds__(NT, 1) void scan_kernel(const ScanArgs a)
{
    __shared__ __attribute__((aligned(16))) char sm[LDS_BYTES];
    if (PASS3) {
        if (TP) scan_segment<true, true>(a, sm, false);
        scan_segment<true, false>(a, sm, false);
    } else {
        if (a.seg0_out) scan_segment<true, false>(a, sm, true);
        scan_segment<false, TP>(a, sm, true);
    }
}

// Pass 2: entering states of segments 2.. of every sequence,
// S_start(j+1) = M_j S_start(j) + R_j, for one 16-column slice of one
// (sequence, head).  The 8 slices of a unit run on one XCD (they read the
// same M_j).  fp32 matrix instructions (16x16x4, exact fp32 products, fp32
// sums): wave w owns rows 16w..16w+15 of the slice.  The slice of S is kept in
// LDS in accumulator layout (lane group g: rows 4g..4g+3 of a row tile); with
// the sum index ordered so that step (t, i) of a product takes rows 16t + 4g + i,
// a tile in accumulator layout is directly the B operand of the next product,
// and the A operand of lane (row, g) is the float4 M[row][16t + 4g .. +3].
__global__ __launch_bounds__(512) void combine_kernel(const ScanArgs a)
{
    __shared__ f32x4 xs[8][64];  // S slice: row tile, lane
    const int bid = blockIdx.x;
    const int slice = (bid >> 3) & 7;
    const int64_t unit = static_cast<int64_t>(bid >> 6) * 8 + (bid & 7);
    const int H = a.H;
    if (unit >= a.n_seq * H) return;
    const int64_t n = unit / H;
    const int h = static_cast<int>(unit - n * H);
    int64_t z0, nseg;  // z0: the sequence's first workspace slot
    if (!a.cu_seqlens) {
        nseg = a.nseg_dense;
        z0 = n * nseg;
    } else {
        nseg = static_cast<int64_t>(a.seg_first[n + 1]) - a.seg_first[n];
        z0 = a.ws_first[n];
    }
    if (nseg < 3) return;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int col = 16 * slice + (lane & 15), g = lane >> 4;
    const int crow = 16 * wave + 4 * g;          // accumulator rows crow..crow+3
    const int arow = 16 * wave + (lane & 15);    // A-operand row
    {
        const float* src = a.ws_start + ((z0 + 1) * H + h) * SS;
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = src[(crow + i) * kDim + col];
        xs[wave][lane] = x;
    }
    // M_j rows and R_j of the first step; each step requests the next one's
    float4 mc[8];
    f32x4 rc;
    auto load = [&](int64_t jj, float4 (&m)[8], f32x4& r) {
        const float* M = a.ws_maps + (((z0 + jj) * H + h) * 2) * SS;
#pragma unroll
        for (int t = 0; t < 8; ++t) m[t] = *reinterpret_cast<const float4*>(M + arow * kDim + 16 * t + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = M[SS + (crow + i) * kDim + col];
    };
    load(1, mc, rc);
    __syncthreads();
    for (int64_t jj = 1; jj + 1 < nseg; ++jj) {
        float4 mn[8];
        f32x4 rn;
        if (jj + 2 < nseg) load(jj + 1, mn, rn);
        f32x4 c = rc;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4 b = xs[t][lane];
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(mc[t].x, b[0], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(mc[t].y, b[1], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(mc[t].z, b[2], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(mc[t].w, b[3], c, 0, 0, 0);
        }
        __syncthreads();  // every wave has read the slice
        float* dst = a.ws_start + ((z0 + jj + 1) * H + h) * SS;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(crow + i) * kDim + col] = c[i];
        xs[wave][lane] = c;
        __syncthreads();
        if (jj + 2 < nseg) {
#pragma unroll
            for (int t = 0; t < 8; ++t) mc[t] = mn[t];
            rc = rn;
        }
    }
}

// Packed sequences: the segment length and the first segment index of every
// sequence, seg_first[n] = sum_{m < n} max(1, ceil(len_m / L)), with L stored
// in seg_first[n_seq + 1].  One workgroup.
//
// L is chosen among seg_max and the powers of two below it down to seg_min
// by the time it predicts for the two scan passes.  Pass 1 runs every segment
// but the last of each sequence, all exactly L tokens long: it takes
// ceil(segments * H / CUs) rounds of L tokens.  Pass 3 runs every segment and
// takes about the larger of its work spread over the CUs and its longest
// segment.  Relative to a pass-3 chunk that forms T and P, a pass-1 chunk
// costs about 0.9, or 1.07 when it also keeps T and P (tp), and a pass-3
// chunk that reuses them 0.6.  Short segments balance the CUs but add pass-1
// work (every boundary is one more map); the lengths are only known here, on
// the device.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* cu, int64_t n_seq,
                                                    int64_t seg_max, int64_t seg_min, int64_t H,
                                                    int64_t n_cu, int tp, int32_t* seg_first,
                                                    int32_t* ws_first, int32_t* seg_order)
{
    constexpr int kCand = 6;
    __shared__ int64_t part[1024];
    __shared__ double work1[kCand][32];
    __shared__ int64_t longest_part[32];
    __shared__ int64_t chosen;
    const int tid = threadIdx.x;
    const int64_t lo = n_seq * tid / 1024, hi = n_seq * (tid + 1) / 1024;
    int64_t cand[kCand];
    int nc = 0;
    cand[nc++] = seg_max;
    {
        int64_t L = 64;
        while (L * 2 < seg_max) L *= 2;  // the largest power of two below seg_max
        for (; L >= seg_min && L >= 64 && nc < kCand; L /= 2) cand[nc++] = L;
    }
    // per candidate: the number of pass-1 segments (all but each sequence's last)
    double w1[kCand];
    int64_t longest = 0, total = 0;
    for (int c = 0; c < kCand; ++c) w1[c] = 0.0;
    for (int64_t m = lo; m < hi; ++m) {
        const int64_t len = static_cast<int64_t>(cu[m + 1]) - cu[m];
        longest = len > longest ? len : longest;
        total += len;
        for (int c = 0; c < nc; ++c)
            if (len > cand[c]) w1[c] += static_cast<double>((len - 1) / cand[c]);
    }
    // reduce over the workgroup: wave sums through LDS
    const int wave = tid >> 6, lane = tid & 63;
    for (int off = 32; off > 0; off >>= 1) {
        for (int c = 0; c < nc; ++c) w1[c] += __shfl_xor(w1[c], off);
        const int64_t lo2 = __shfl_xor(longest, off);
        longest = lo2 > longest ? lo2 : longest;
        total += __shfl_xor(total, off);
    }
    if (lane == 0) {
        for (int c = 0; c < nc; ++c) work1[c][wave] = w1[c];
        longest_part[wave] = longest;
        part[wave] = total;
    }
    __syncthreads();
    if (tid == 0) {
        int64_t lg = 0, tot = 0;
        for (int w = 0; w < 16; ++w) {
            lg = longest_part[w] > lg ? longest_part[w] : lg;
            tot += part[w];
        }
        const double per_cu3 = static_cast<double>(tot) * H / n_cu;
        double best = 0.0;
        int64_t pick = cand[0];
        for (int c = 0; c < nc; ++c) {
            double sum1 = 0.0;
            for (int w = 0; w < 16; ++w) sum1 += work1[c][w];
            const double p1 = ceil(sum1 * H / n_cu) * static_cast<double>(cand[c]);
            // with T/P reuse the mapped tokens (sum1 segments of L) cost 0.6 in pass 3
            const double saved3 = tp ? 0.4 * sum1 * static_cast<double>(cand[c]) * H / n_cu : 0.0;
            const double p3 = fmax(per_cu3 - saved3, static_cast<double>(cand[c] < lg ? cand[c] : lg));
            const double est = (tp ? 1.07 : 0.9) * p1 + p3;
            if (c == 0 || est < best) {
                best = est;
                pick = cand[c];
            }
        }
        chosen = pick;
    }
    __syncthreads();
    const int64_t seg_len = chosen;
    auto count = [&](int64_t m) {
        const int64_t len = static_cast<int64_t>(cu[m + 1]) - cu[m];
        const int64_t c = (len + seg_len - 1) / seg_len;
        return c > 1 ? c : int64_t(1);
    };
    int64_t s = 0;
    for (int64_t m = lo; m < hi; ++m) s += count(m);
    part[tid] = s;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int64_t x = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += x;
        __syncthreads();
    }
    int64_t run = part[tid] - s;  // exclusive prefix
    for (int64_t m = lo; m < hi; ++m) {
        seg_first[m] = static_cast<int32_t>(run);
        run += count(m);
    }
    if (tid == 1023) {
        seg_first[n_seq] = static_cast<int32_t>(part[1023]);
        seg_first[n_seq + 1] = static_cast<int32_t>(seg_len);
    }
    __syncthreads();
    const int64_t n_act = part[1023];
    __syncthreads();
    // workspace slots: only sequences of two or more segments use any
    int64_t s2 = 0;
    for (int64_t m = lo; m < hi; ++m) {
        const int64_t c = count(m);
        s2 += c > 1 ? c : 0;
    }
    part[tid] = s2;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int64_t x = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += x;
        __syncthreads();
    }
    int64_t run2 = part[tid] - s2;
    for (int64_t m = lo; m < hi; ++m) {
        const int64_t c = count(m);
        ws_first[m] = static_cast<int32_t>(run2);
        run2 += c > 1 ? c : 0;
    }
    if (tid == 1023) ws_first[n_seq] = static_cast<int32_t>(part[1023]);

    // Launch order: segments by decreasing chunk count (a counting sort; the
    // order within one count is whatever the atomics give, which changes no
    // result: every segment is computed the same way wherever it runs).
    constexpr int NB = 2048;  // chunk-count buckets; longer segments share the top one
    __shared__ int hist[NB], start[NB];
    for (int b = tid; b < NB; b += 1024) hist[b] = 0;
    __syncthreads();
    auto bucket_of = [&](int64_t z) {
        int64_t lo2 = 0, hi2 = n_seq;  // seg_first[lo2] <= z < seg_first[hi2]
        while (hi2 - lo2 > 1) {
            const int64_t mid = (lo2 + hi2) >> 1;
            if (seg_first[mid] <= z) lo2 = mid;
            else hi2 = mid;
        }
        const int64_t len = static_cast<int64_t>(cu[lo2 + 1]) - cu[lo2];
        const int64_t j = z - seg_first[lo2];
        const int64_t nseg = static_cast<int64_t>(seg_first[lo2 + 1]) - seg_first[lo2];
        const int64_t tokens = nseg == 1 ? len : (j == nseg - 1 ? len - j * seg_len : seg_len);
        const int64_t chunks = (tokens + 63) / 64;
        return static_cast<int>(chunks < NB ? chunks : NB - 1);
    };
    for (int64_t z = tid; z < n_act; z += 1024) atomicAdd(&hist[bucket_of(z)], 1);
    __syncthreads();
    if (tid == 0) {
        int run3 = 0;
        for (int b = NB - 1; b >= 0; --b) {
            start[b] = run3;
            run3 += hist[b];
        }
    }
    __syncthreads();
    for (int64_t z = tid; z < n_act; z += 1024) {
        const int r = atomicAdd(&start[bucket_of(z)], 1);
        seg_order[r] = static_cast<int32_t>(z);
    }
}

// ---------------- host side

static_assert(TP_BYTES == kTpBytes, "the plan sizes the T/P images of this kernel");
static_assert(CH == kChunk && SS == kStateFloats, "the plan's chunk and state sizes");

}  // namespace

// Segment length: enough segments to give every CU about one segment of the
// total work, never shorter than kMinSegment tokens (or the forced length).
//
// Dense input: the first segment of each sequence runs with outputs in pass
// 1, beside the maps of the others, so a sequence takes one segment more for
// the same number of workgroups per pass.  Pass 1 also keeps the split T and
// P of every chunk it maps (32 KiB each) in the fastest plan.  A pass-3 chunk
// that reuses them costs about 3/5 of one that forms them, so the last
// segment (which pass 1 does not map) gets about 3/5 of the others' length;
// the first segment, with outputs in pass 1, costs about as much per chunk as
// a mapped one and is as long.  (Timed: 32 heads x 32,768 tokens, equal
// segments of 3,840 and a last one of 2,048 beat a first segment 17/16 as
// long by 1%, and lengths 64 tokens shorter or longer by 5% and 3%.)  Without
// the images a chunk with outputs costs about 8/7 of a map chunk, and the
// first segment is 7/8 as long instead.
//
// Packed input: the plan kernel picks the length on the device, between seg
// and seg_min; grid and workspace are sized for the shortest candidate.
// Workspace slots: dense, one per segment; packed, only the segments of
// sequences cut in two or more, fewer than 2 * T_total / seg_min of them
// (such a sequence is longer than a segment, so its count is below twice its
// length over the segment length).
hipError_t launch_prefill_scan(const void* q, const void* k, const void* v, const void* beta,
                               const float* log_alpha, const int32_t* cu_seqlens, int64_t n_seq,
                               int64_t T, int64_t H, const StateRefs& st, float* o, bool raw,
                               int64_t short_max, const PrefillPlan& plan, void* ws, int n_cu,
                               hipStream_t stream)
{
    const int64_t units = n_seq * H;
    if (units <= 0) return hipSuccess;
    ScanArgs a = {};
    a.q = static_cast<const bf16_t*>(q);
    a.k = static_cast<const bf16_t*>(k);
    a.v = static_cast<const bf16_t*>(v);
    a.beta = static_cast<const bf16_t*>(beta);
    a.log_alpha = log_alpha;
    a.cu_seqlens = cu_seqlens;
    a.T = T;
    a.n_seq = n_seq;
    a.H = static_cast<int>(H);
    a.st = st;
    a.o = o;
    a.raw = raw ? 1 : 0;
    a.short_max = short_max > 0 ? short_max : -1;  // -1: no sequence is skipped (lengths are >= 0)
    const dim3 block(NT);
    hipError_t e;

    if (!plan.segmented) {
        // one segment per sequence: pass 3 alone from the given initial states
        a.seg_len = 0;
        a.nseg_dense = 1;
        a.n_segs = n_seq;
        a.seg_first = nullptr;
        hipLaunchKernelGGL((scan_kernel<true, false>), dim3(static_cast<unsigned>(units)), block, 0,
                           stream, a);
        e = hipGetLastError();
        report("prefill scan launch", e);
        return e;
    }

    a.seg_len = plan.seg;
    a.seg0_len = plan.seg0;
    a.seg0_out = cu_seqlens ? 0 : 1;
    a.n_segs = plan.n_segs;
    a.nseg_dense = plan.nseg_dense;
    char* w = static_cast<char*>(ws);
    if (cu_seqlens) {
        a.seg_first = reinterpret_cast<int32_t*>(w);             // [n_seq + 2]
        a.ws_first = a.seg_first + n_seq + 2;                     // [n_seq + 1]
        a.seg_order = a.ws_first + n_seq + 1;                     // [n_segs]
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, n_seq, plan.seg,
                           plan.seg_min, H, static_cast<int64_t>(n_cu), plan.tp ? 1 : 0,
                           const_cast<int32_t*>(a.seg_first), const_cast<int32_t*>(a.ws_first),
                           const_cast<int32_t*>(a.seg_order));
        e = hipGetLastError();
        report("segment plan launch", e);
        if (e != hipSuccess) return e;
    }
    a.ws_maps = reinterpret_cast<float*>(w + plan.plan_bytes);
    a.ws_start = a.ws_maps + static_cast<size_t>(plan.slots) * H * 2 * SS;
    if (plan.tp) a.ws_tp = reinterpret_cast<char*>(a.ws_start + static_cast<size_t>(plan.slots) * H * SS);

    const dim3 grid(static_cast<unsigned>(plan.n_segs * H));
    if (plan.tp) hipLaunchKernelGGL((scan_kernel<false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((scan_kernel<false, false>), grid, block, 0, stream, a);
    e = hipGetLastError();
    report("segment map launch", e);
    if (e != hipSuccess) return e;
    const dim3 cgrid(static_cast<unsigned>((units + 7) / 8 * 64));
    hipLaunchKernelGGL(combine_kernel, cgrid, dim3(512), 0, stream, a);
    e = hipGetLastError();
    report("segment combine launch", e);
    if (e != hipSuccess) return e;
    if (plan.tp) hipLaunchKernelGGL((scan_kernel<true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((scan_kernel<true, false>), grid, block, 0, stream, a);
    e = hipGetLastError();
    report("prefill scan launch", e);
    return e;
}

}  // namespace kda
