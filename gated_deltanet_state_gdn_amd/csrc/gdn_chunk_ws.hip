// Chunked gated delta rule (replay and prefill) for gfx950 / CDNA4.
//
// The recurrence (Gated DeltaNet, as replayed by Tail-Replay over the last r tokens
// of a matched prefix from a zero state; gist.science technical summary,
// "Mecanismos Principais"):
//     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,   o_t = scale S_t^T q_t
// is evaluated in chunks of C = 64 tokens.  For one chunk with incoming state S:
//     H_i  cumulative log-gate since the last a = 0 token,  e_i = exp(H_i) (0 after a reset)
//     G_ij = exp(H_i - H_j) if no reset in (j, i], else 0             (j <= i)
//     A    = strict_lower(diag(b) (K K^T o G))
//     (I + A) U = Y,  Y = diag(b) (V - diag(e) K S)                     (UT transform)
//     O    = diag(scale e) Q S + P U,   P = scale lower(Q K^T o G)  (diagonal included)
//     S   <- e_last S + K^T diag(G_last,.) U
// which equals the token recurrence exactly in exact arithmetic.  The triangular
// solve runs as forward substitution over 16-row blocks,
//     U_b = Z_b + (T_bb - I) Z_b,   Z_b = Y_b - sum_{j<b} A_bj U_j,   T_bb = (I + A_bb)^{-1}.
//
// Work decomposition: one workgroup per (sequence, v-head, d_v block), split into two
// roles that run concurrently on two LDS chunk buffers:
//   * state waves (one per 16-column tile of S): the sequential pass over the chunks.
//     S never leaves their MFMA accumulators; the columns of S evolve independently
//     because (I - b k k^T) acts on the d_k side only, so they exchange nothing.
//     The outputs are formed transposed (O^T = S^T Q^T + U^T P^T), which puts four
//     consecutive d_v entries of one token in a lane: one vector store per 16 tokens.
//   * eight prep waves: everything that does not depend on S, one chunk ahead -- the
//     chunk's K and Q (and, for bf16 inputs, V) in LDS (all eight), the Gram products
//     forming -A and P and the diagonal-block inverses (seven), the gate scan (one).
// The state waves keep S / sig instead of S, sig being the product of the chunk decays
// since the last renormalisation, so the per-chunk decay e_last costs no pass over S.
// One workgroup barrier per chunk hands a prepared buffer to the state waves; the
// prep waves order their own steps with a counter in LDS.
//
// Global memory is read and written through buffer resources rebased at every chunk:
// 32-bit offsets, no per-element 64-bit address arithmetic, and the hardware range
// check returns zero for the rows past the end of a sequence's last chunk (and drops
// stores there).  Zero rows are inert: their g and b are 0, so they neither decay nor
// write the state.
//
// Precision (bf16 inputs, fp32 state): every matrix product has fp16 operands and fp32
// accumulation.  q and k are converted to fp16 exactly when staged (they are L2-normalised,
// so well inside fp16's range); S, U, P, A_bj, T_bb - I and Z are rounded to fp16 once
// (11 significant bits against bf16's 8).  The bf16 layout this replaces needed hi + lo
// pairs for S, U and P (1.7x the matrix products) and still left a 2-4x larger state
// error, from the bf16 rounding of S in K S and of A_bj, T_bb - I and Z.  v, the gates, b
// and the unit diagonal of the solve stay fp32.  Range: the stored state S / sig is kept within 64 |S| (sig >= 2^-6),
// so state entries up to ~10^3 fit fp16.  fp32 inputs use fp32 MFMA throughout.
//
// Matrix-core layout used (16x16 MFMA): lane l supplies row l%16 of A and column
// l%16 of B; element j of lane group l/16 in A pairs with element j of the same
// lane group in B; the accumulator holds D[4*(l/16)+i][l%16] in element i.  A
// fragment whose contraction indices follow the accumulator rows lets a D tile be
// used directly as a B operand (S in K S, Z/U in the solve, U in K^T U) and, read
// the other way, as an A operand (S^T in S^T Q^T, U^T in U^T P^T).
#include <atomic>
#include <type_traits>

#include "gdn_common.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 h16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 h16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 h16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __amdgpu_buffer_rsrc_t Rsrc;

constexpr int CH = 64;       // chunk length (tokens)
constexpr int kOrderSeqs = 256;   // most packed sequences a launch orders by length
constexpr int NPW = 8;       // prep waves per workgroup

// Two floats to a bf16 pair (round to nearest even), the first in the low half: the
// outputs o of the bf16 path.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// Two floats to an fp16 pair (round to nearest even, v_cvt_pk_f16_f32), the first in the
// low half: every matrix operand of the bf16 path.
__device__ __forceinline__ uint32_t pk_h(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, h16x2));
}
// A bf16 pair as an fp16 pair: exact for magnitudes in [2^-14, 65504], the range the
// L2-normalised q and k of a Gated DeltaNet layer live in (smaller ones round to fp16
// subnormals).
__device__ __forceinline__ uint32_t bf2_to_h2(uint32_t p) {
    return pk_h(__uint_as_float(p << 16), __uint_as_float(p & 0xffff0000u));
}

// ---------------------------------------------------------------- policies
struct PolF32 {
    static constexpr bool kBF16 = false;
    static constexpr int KB = 16;    // contraction length of one fragment step
    typedef float E;                 // element type of q/k/v and of LDS operands
    typedef f32x4 Frag;
};
// bf16 inputs: q, k, v stored as bf16; every matrix operand an fp16 value (q and k
// converted exactly when staged, the fp32 intermediates rounded once), fp32 accumulation.
struct PolBF16 {
    static constexpr bool kBF16 = true;
    static constexpr int KB = 32;
    typedef uint16_t E;
    typedef h16x8 Frag;
};

__device__ __forceinline__ f32x4 mma(f32x4 c, f32x4 a, f32x4 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}
__device__ __forceinline__ f32x4 mma(f32x4 c, h16x8 a, h16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- global memory
// Untyped buffer over [base, base + bytes): loads past the end return 0 and stores past
// it are dropped.
__device__ __forceinline__ Rsrc make_rsrc(const void *base, int64_t bytes) {
    const int32_t n = bytes <= 0 ? 0 : (int32_t)(bytes < 0x7fffffffLL ? bytes : 0x7fffffffLL);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
// One element of q/k/v in a register, kept in its storage width until it is used (a
// widening right after the load would make the loop wait for it early).
template <class P> struct Raw {
    typedef typename std::conditional<P::kBF16, uint16_t, uint32_t>::type T;
};
template <class P>
__device__ __forceinline__ typename Raw<P>::T load_e(Rsrc r, uint32_t off) {
    if constexpr (P::kBF16) return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
template <class P>
__device__ __forceinline__ float v_at(typename Raw<P>::T v) {
    if constexpr (P::kBF16) return __uint_as_float((uint32_t)v << 16);
    else return __uint_as_float(v);
}

// The lane index, computed afresh where it is called (an opaque all-ones mask keeps the
// compiler from hoisting it out of a loop): inside the chunk loops this costs two vector
// instructions instead of a register held across the whole loop.
__device__ __forceinline__ int fresh_lane() {
    uint32_t m = ~0u;
    asm volatile("" : "+s"(m));
    return (int)__builtin_amdgcn_mbcnt_hi(m, __builtin_amdgcn_mbcnt_lo(m, 0u));
}

// A value that is the same in every lane of the wave, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------- LDS layouts
// Operand matrices (K, Q) are row-major with RB-byte rows of 16-byte chunks and no
// padding: logical chunk c of row r sits at chunk c ^ swz(r).  bf16 columns are permuted
// inside every 32-column block so that one chunk holds a whole fragment: logical chunk
// 4 kb + g carries columns 32 kb + {4g..4g+3, 16+4g..16+4g+3}, the contraction indices
// that pair with accumulator rows 4g + i of two 16-row tiles; an aligned group of four
// columns is always 8 contiguous bytes.  fp32 keeps the natural order (logical chunk
// 4 kb + g = columns 16 kb + 4g .. 4g+3).
// The swizzle for 256-byte rows puts the three low row bits, reversed, on chunk bits
// 3..1.  Chosen by measurement (the LDS bank-conflict counter over every XOR swizzle of
// the low four row bits): it is free of conflicts for 16-byte row fragments (16 rows,
// one logical chunk per 16 lanes) and keeps the 8-byte transposing reads of K^T
// fragments (4 rows x 4 chunks) at the rate of an unswizzled 8-byte read; swapping the
// two 2-bit halves of the row index, the obvious choice, doubles the fragment reads'
// cost.  128-byte rows keep a swap-style swizzle.
template <int RB>
__device__ __forceinline__ int swz(int r) {
    return RB == 256 ? (((r & 1) << 3) | ((r & 2) << 1) | ((r & 4) >> 1))
                     : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}
template <int RB>
__device__ __forceinline__ int chunk_at(int r, int c) { return r * RB + 16 * (c ^ swz<RB>(r)); }

// A-operand fragment (or B = M^T): lane l gives row r0 + l%16 and logical chunk
// 4 kb + l/16 (r0 a multiple of 16).
template <int RB, class F>
__device__ __forceinline__ F frag_sw(const char *M, int r0, int kb, int lane) {
    return __builtin_bit_cast(
        F, *reinterpret_cast<const u32x4 *>(M + chunk_at<RB>(r0 + (lane & 15), 4 * kb + (lane >> 4))));
}
// The same addresses with one XOR per k-block.  The swizzle depends only on the row's
// low four bits, which r0 (a multiple of 16) leaves alone, and the logical chunk
// 4 kb + g is 4 kb XOR g, so
//     chunk_at(r0 + l%16, 4 kb + l/16) = r0 RB + (fo ^ 64 kb),
//     fo = (l%16) RB + 16 ((l/16) ^ swz(l%16)),
// since every term stays below RB (no carries).  An offset that is a multiple of 256 (a
// chunk buffer) may be added to fo before the XOR.
template <int RB>
__device__ __forceinline__ uint32_t frag_off(int lane) {
    const int r = lane & 15;
    return (uint32_t)(r * RB + 16 * ((lane >> 4) ^ swz<RB>(r)));
}
template <class F>
__device__ __forceinline__ F frag_at(const char *p) {
    return __builtin_bit_cast(F, *reinterpret_cast<const u32x4 *>(p));
}
// bf16 fragment of K^T for one 16x16x32 product, read transposed from the row-major K:
// lane l gets K[32 kb + {4 (l/16) + i, 16 + 4 (l/16) + i}][16 rt + l%16], i = 0..3.  The
// transposing read hands lane n of every 16-lane group column n%4 of rows
// {n/4, n/4 + 4, n/4 + 8, n/4 + 12} of the 16 x 4 block whose row m is the 8 bytes lane m
// points at; lane m = 4 y + x of group g points at token 32 kb + 4 g + y (+16 for the
// second half), columns 16 rt + 4 x .. +3.
typedef __attribute__((ext_vector_type(4))) short i16x4;
template <int RB>
__device__ __forceinline__ h16x8 frag_kt(const char *K, int rt, int kb, int lane) {
    const int m = lane & 15;
    const int row = 32 * kb + 4 * (lane >> 4) + (m >> 2);
    const char *p = K + chunk_at<RB>(row, 4 * (rt >> 1) + (m & 3)) + 8 * (rt & 1);
    typedef __attribute__((address_space(3))) i16x4 *lds_i16x4;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)p);
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(p + 16 * RB));
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    return __builtin_bit_cast(h16x8, u32x4{ua.x, ua.y, ub.x, ub.y});
}
// Lane part of the transposing reads' addresses (frag_kt, frag_v), by the argument of
// frag_off: with m = l%16 and row 4 (l/16) + m/4 inside a 16-row block,
//     chunk_at(R0 + row, 4 j + m%4) + 8 h = R0 RB + (to ^ 64 j) + 8 h,
//     to = row RB + 16 ((m%4) ^ swz(row)),
// for R0 a multiple of 16 (32 kb for K^T rows, 16 tt for V rows).
template <int RB>
__device__ __forceinline__ uint32_t tr_off(int lane) {
    const int m = lane & 15;
    const int row = 4 * (lane >> 4) + (m >> 2);
    return (uint32_t)(row * RB + 16 * ((m & 3) ^ swz<RB>(row)));
}
// frag_kt from tr_off: K points at the K rows of a chunk buffer (tob = to + buffer offset)
template <int RB>
__device__ __forceinline__ h16x8 frag_kt_at(const char *K, uint32_t tob, int rt, int kb) {
    const char *p = K + 32 * kb * RB + (tob ^ (uint32_t)(64 * (rt >> 1))) + 8 * (rt & 1);
    typedef __attribute__((address_space(3))) i16x4 *lds_i16x4;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)p);
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(p + 16 * RB));
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    return __builtin_bit_cast(h16x8, u32x4{ua.x, ua.y, ub.x, ub.y});
}
// V values of one 16-row tile in the accumulator layout, from the bf16 V rows staged in the
// same permuted, swizzled layout as K: lane l gets V[16 tt + 4 (l/16) + i][16 ct + l%16],
// i = 0..3, as bf16 pairs (element i in half i%2 of word i/2).  One transposing read: lane
// m = 4 y + x of group g points at row 16 tt + 4 g + y, columns 16 ct + 4 x .. +3.
template <int RB>
__device__ __forceinline__ u32x2 frag_v(const char *V, int ct, int tt, int lane) {
    const int m = lane & 15;
    const int row = 16 * tt + 4 * (lane >> 4) + (m >> 2);
    const char *p = V + chunk_at<RB>(row, 4 * (ct >> 1) + (m & 3)) + 8 * (ct & 1);
    typedef __attribute__((address_space(3))) i16x4 *lds_i16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)p));
}
// frag_v from vo = tr_off ^ 64 (ct/2) + 8 (ct%2) + buffer offset (V: the staged V rows)
template <int RB>
__device__ __forceinline__ u32x2 frag_v_at(const char *V, uint32_t vo, int tt) {
    typedef __attribute__((address_space(3))) i16x4 *lds_i16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(V + 16 * tt * RB + vo)));
}
// fp32 fragment of M^T (the rows of M are the contraction index): lane l gives column
// c0 + l%16 and rows 16 kb + 4 (l/16) + i.
template <int RB>
__device__ __forceinline__ f32x4 frag_cols_f32(const char *M, int c0, int kb, int lane) {
    const int col = c0 + (lane & 15);
    f32x4 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * kb + 4 * (lane >> 4) + i;
        f[i] = *reinterpret_cast<const float *>(M + chunk_at<RB>(row, col >> 2) + 4 * (col & 3));
    }
    return f;
}

// The small operand tiles are stored in fragment order: the lane that reads a fragment
// finds it at 16 (or 8) bytes times its lane index, and the lane that writes it uses the
// same index, since producer and consumer share the A-operand layout (lane l: row l%16,
// columns 4 (l/16) .. +3 of a 16x16 tile).  Consecutive lanes then touch consecutive
// bytes, which the LDS serves without bank conflicts (a row-major layout with 32- or
// 64-byte rows measured 2.3e7 and 1.7e7 conflict cycles per 36-layer launch).
//
// bf16-path tile pairs: the 16 x 32 block (16-row block ti, 32-column block kb) of a
// 64x64 lower-triangular matrix as one 16-byte fragment per lane: columns 4 (l/16) .. +3
// of tile (ti, 2kb), then of tile (ti, 2kb+1), of row l%16.
// Pair index of (ti, kb), kb <= ti/2:  0:(0,0) 1:(1,0) 2:(2,0) 3:(2,1) 4:(3,0) 5:(3,1).
__device__ __forceinline__ int dt_index(int ti, int kb) { return ti < 2 ? ti : 2 * ti - 2 + kb; }
__device__ __forceinline__ h16x8 frag_dt(const char *T, int pair, int lane) {
    return __builtin_bit_cast(h16x8, *reinterpret_cast<const u32x4 *>(T + pair * 1024 + 16 * lane));
}

// 16x16 tiles (T_bb - I; for fp32 inputs also -A and P), one 4-element fragment per lane;
// lower tile (ti, tj) of a 64x64 matrix at ti*(ti+1)/2 + tj.
__device__ __forceinline__ int tri_index(int ti, int tj) { return ti * (ti + 1) / 2 + tj; }
// Operands of a 16x16x16 product (4 contraction indices per lane), for the products
// whose other half would be zero: the first tile of a tile pair and a 16x16 tile, both
// in the A-operand layout (lane l: row l%16, columns 4 (l/16) .. +3).
__device__ __forceinline__ u32x2 frag_dt_first(const char *T, int pair, int lane) {
    return *reinterpret_cast<const u32x2 *>(T + pair * 1024 + 16 * lane);
}
__device__ __forceinline__ u32x2 frag_t16(const uint16_t *T, int tile, int lane) {
    return *reinterpret_cast<const u32x2 *>(T + tile * 256 + 4 * lane);
}
__device__ __forceinline__ f32x4 frag_tile(const float *T, int tile, int lane) {
    return *reinterpret_cast<const f32x4 *>(T + tile * 256 + 4 * lane);
}

// ---------------------------------------------------------------- register operands
// Two accumulator tiles (16 contraction rows each) as one fp16 operand.
__device__ __forceinline__ h16x8 bfrag(const f32x4 &t0, const f32x4 &t1) {
    const u32x4 u = {pk_h(t0[0], t0[1]), pk_h(t0[2], t0[3]), pk_h(t1[0], t1[1]), pk_h(t1[2], t1[3])};
    return __builtin_bit_cast(h16x8, u);
}
// One accumulator tile (16 contraction rows) as the B operand of a 16x16x16 product.
__device__ __forceinline__ u32x2 bfrag16(const f32x4 &t) {
    return u32x2{pk_h(t[0], t[1]), pk_h(t[2], t[3])};
}
__device__ __forceinline__ f32x4 mma16(f32x4 c, u32x2 a, u32x2 b) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h16x4, a),
                                                 __builtin_bit_cast(h16x4, b), c, 0, 0, 0);
}

// Workgroup barrier that orders LDS only: global loads stay in flight across it
// (a full __syncthreads also waits for every outstanding global load).
__device__ __forceinline__ void sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Bounded wait until an LDS counter reaches `target`; an expired wait only costs wrong
// results (flagged in the status word), never a hang.
__device__ __forceinline__ void lds_wait_ge(const int *ctr, int target, int *fail) {
    int spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1 << 24)) {
            *fail = 1;
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier among the prep waves only: each wave adds 1 to an LDS counter and waits
// until every prep wave has; the target grows by NPW per use, so the counter is never
// reset.  The wait is bounded: a wave that never arrived would only cost wrong results
// (flagged in the status word), never a hang.
__device__ __forceinline__ void prep_sync(int *ctr, int &target, int lane, int *fail) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    target += NPW;
    if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    int spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1 << 24)) {
            *fail = 1;
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- LDS plan
// Two chunk buffers (the state waves read one while the prep waves fill the other),
// then a few words.  fp32 inputs with d_k = 128 and outputs would need 180 KB that way
// (two 32 KB K and Q copies per buffer), more than a compute unit's 160 KB: there Q has
// one buffer of its own, which the prep waves refill for the next chunk only once every
// state wave has finished its Q S products of the current one (an LDS counter).
template <int DK, int W, class P, bool WITH_O>
struct Lds {
    typedef typename P::E E;
    static constexpr int RBK = DK * (int)sizeof(E);          // K / Q row bytes
    static constexpr int RBV = W * 2;                          // V row bytes (bf16 inputs)
    static constexpr int TILE = 256 * (int)sizeof(E);          // one 16x16 tile
    static constexpr int NTA = P::kBF16 ? 6 : 10;              // tile pairs (bf16) / tiles (fp32)
    static constexpr int UNIT = P::kBF16 ? 1024 : TILE;
    static constexpr bool Q1 = WITH_O && !P::kBF16 && DK == 128;   // single Q buffer
    // gate rows: H (log2(e) units for bf16 inputs), e sig, b, G_last / sig, scale e sig,
    // rho (int), the chunk's state-scale words (renormalisation factor, sig after the
    // chunk), and for fp32 inputs the lo part of H; 8 rows keep K at a 1 KB boundary
    static constexpr int oGate = 0;
    static constexpr int oK = 8 * CH * 4;
    static constexpr int oQ = oK + CH * RBK;
    // V of the block's column range (bf16 inputs; fp32 inputs read V from global memory)
    static constexpr int oV = oQ + ((WITH_O && !Q1) ? CH * RBK : 0);
    static constexpr int oA = oV + (P::kBF16 ? CH * RBV : 0);  // -A
    static constexpr int oT = oA + NTA * UNIT;                   // 4 tiles T_bb - I
    static constexpr int oPh = oT + 4 * TILE;                    // P
    static constexpr int BUF = oPh + (WITH_O ? NTA * UNIT : 0);
    static constexpr int oQ1 = 2 * BUF;                          // the single Q buffer
    static constexpr int oMisc = oQ1 + (Q1 ? CH * RBK : 0);
    static constexpr int bytes = oMisc + 64;
    // Q rows of the chunk in buffer `buf`
    __device__ static const char *q_rows(const char *smem, const char *buf) {
        return Q1 ? smem + oQ1 : buf + oQ;
    }
};

// ---------------------------------------------------------------- prep-wave pieces
// Gates of one chunk, one token per lane: reset-aware inclusive scan of the log-gates
// (H = sum of g since the last alpha = 0 token), e = exp(H) (0 once a reset occurred),
// G_last = exp(H_63 - H) (0 before the chunk's last reset), rho = last reset position.
//
// For fp32 inputs (COMP) H is carried as an unevaluated sum h + lo of two floats: every
// addition of the scan is a two-sum (Knuth) whose rounding error goes into lo, and the
// differences H_i - H_j behind every G_ij are taken as (h_i - h_j) + (lo_i - lo_j),
// accurate to the size of the difference rather than of H.  A plain fp32 scan loses
// ulp(|H|) there: under fast decay |H| reaches a few hundred within a chunk, so G entries
// near 1 (the last tokens' weights in the state update) are off by ~1e-5; in a partial
// last chunk the scan even sums H_63 and H_{n-1} (equal: the rows past the window add
// zeros) in different orders, so the newest token's weight, exactly 1, comes out as
// 1 +- 1.5e-5 -- beyond the fp32 inputs' 1e-5 tolerance, far inside bf16's 3e-3, so
// bf16 inputs keep the plain scan.
struct Gates {
    float h, lo, e, b, l;
    int rho;
};
template <bool COMP>
__device__ __forceinline__ Gates gate_scan(float gv, float bv, int lane) {
    const bool reset = gv == -__builtin_inff();
    float hv = reset ? 0.f : gv, lv = 0.f;
    int seg = reset ? 1 : 0;
    int rho = reset ? lane : -1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float ho = __shfl_up(hv, off);
        const float lo = COMP ? __shfl_up(lv, off) : 0.f;
        const int so = __shfl_up(seg, off);
        const int ro = __shfl_up(rho, off);
        if (lane >= off) {
            if (!seg) {
                const float sm = hv + ho;
                if constexpr (COMP) {
                    const float bp = sm - hv;
                    const float err = (hv - (sm - bp)) + (ho - bp);
                    lv = lv + lo + err;
                }
                hv = sm;
            }
            seg |= so;
            rho = ro > rho ? ro : rho;
        }
    }
    const float hl = __shfl(hv, 63), ll = COMP ? __shfl(lv, 63) : 0.f;
    const int rl = __shfl(rho, 63);
    Gates g;
    g.h = hv;
    g.lo = lv;
    g.e = rho < 0 ? __expf(hv) : 0.f;
    g.b = bv;
    g.l = rl <= lane ? __expf(COMP ? (hl - hv) + (ll - lv) : hl - hv) : 0.f;
    g.rho = rho;
    return g;
}

// One Gram tile (ti, tj) of a chunk, in three stages so that a wave can overlap the
// LDS latency of one tile with the work of the previous one:
//   tile_load  every fragment and gate value the tile needs, issued together;
//   tile_mma   K_tj K_ti^T and K_tj Q_ti^T on the matrix cores;
//   tile_store -A and P = scale lower(Q K^T o G) (fp16 for bf16 inputs) into LDS.
// The products are formed as K_tj K_ti^T and K_tj Q_ti^T, so that element e of lane l is
//     kk[e] = k_{16 tj + 4 (l/16) + e} . k_{16 ti + l%16},
//     qk[e] = k_{16 tj + 4 (l/16) + e} . q_{16 ti + l%16},
// entry (16 ti + l%16, 16 tj + 4 (l/16) + e) of K K^T and of Q K^T: four consecutive
// columns of one row per lane, stored with one vector write.  The -A values are
// returned (for ti == tj: the diagonal block in the A-operand layout).
template <class P, int KBK>
struct TileIn {
    typename P::Frag kj[KBK], ki[KBK], qi[KBK];
    f32x4 hc, lc = {0.f, 0.f, 0.f, 0.f};   // lc, lr: the lo parts of H (fp32 inputs only)
    float hr, lr = 0.f, br;
    int rho;
};
// (tile_load and tile_mma cover the k-blocks [KB0, KB1) of d_k: all of them, or one half
// at a time where a whole tile's fragments would not fit in registers)
template <int DK, class P, bool WITH_O, class L, int KB0 = 0, int KB1 = DK / P::KB>
__device__ __forceinline__ void tile_load(TileIn<P, DK / P::KB> &t, const char *buf, const char *lds, uint32_t bo,
                                          int ti, int tj, int lane) {
    typedef typename P::Frag F;
    const float *gH = reinterpret_cast<const float *>(buf + L::oGate);
    // fragment addresses by frag_off (bo: the chunk buffer's offset in LDS)
    const uint32_t fo = frag_off<L::RBK>(lane);
    const uint32_t fob = fo + bo, qob = L::Q1 ? fo : fob;
    const char *Kb = lds + L::oK, *Qb = lds + (L::Q1 ? L::oQ1 : L::oQ);
#pragma unroll
    for (int kb = KB0; kb < KB1; ++kb) {
        t.kj[kb] = frag_at<F>(Kb + 16 * tj * L::RBK + (fob ^ (64u * kb)));
        t.ki[kb] = frag_at<F>(Kb + 16 * ti * L::RBK + (fob ^ (64u * kb)));
        if constexpr (WITH_O) t.qi[kb] = frag_at<F>(Qb + 16 * ti * L::RBK + (qob ^ (64u * kb)));
    }
    const int rr = 16 * ti + (lane & 15);
    t.hr = gH[rr];
    t.br = gH[2 * CH + rr];
    t.rho = reinterpret_cast<const int *>(gH + 5 * CH)[rr];
    t.hc = *reinterpret_cast<const f32x4 *>(gH + 16 * tj + 4 * (lane >> 4));
    if constexpr (!P::kBF16) {
        t.lr = gH[7 * CH + rr];
        t.lc = *reinterpret_cast<const f32x4 *>(gH + 7 * CH + 16 * tj + 4 * (lane >> 4));
    }
}
template <int DK, class P, bool WITH_O, int KB0 = 0, int KB1 = DK / P::KB>
__device__ __forceinline__ void tile_mma(const TileIn<P, DK / P::KB> &t, f32x4 &kk, f32x4 &qk) {
    if constexpr (KB0 == 0) {
        kk = f32x4{0.f, 0.f, 0.f, 0.f};
        qk = kk;
    }
#pragma unroll
    for (int kb = KB0; kb < KB1; ++kb) {
        kk = mma(kk, t.kj[kb], t.ki[kb]);
        if constexpr (WITH_O) qk = mma(qk, t.kj[kb], t.qi[kb]);
    }
}
template <int DK, class P, bool WITH_O, class L>
__device__ __forceinline__ f32x4 tile_store(char *buf, float hr, float lr_, float br, int rho, f32x4 hc,
                                            f32x4 lc, f32x4 kk, f32x4 qk, int ti, int tj, int lane,
                                            float scale) {
    const int lr = lane & 15, lg = lane >> 4;
    const int rr = 16 * ti + lr;
    f32x4 av, pv, ex;
    // exp(H_i - H_j) of every entry, then a select: no divergent branch (the unused ones
    // may be inf).  bf16 inputs: the gate row holds H log2(e), so one exp2 of the
    // difference (its rounding, ~1e-5 relative under fast decay, is far below the bf16
    // tolerance); fp32 inputs: the difference of the (hi, lo) pairs, then scaled.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (P::kBF16) {
            ex[e] = __builtin_amdgcn_exp2f(hr - hc[e]);
        } else {
            ex[e] = __builtin_amdgcn_exp2f(((hr - hc[e]) + (lr_ - lc[e])) * 1.4426950408889634f);
        }
    }
    // Off-diagonal tiles (ti > tj, known when inlined) lie wholly below the diagonal; when
    // in addition no row's last reset lies at or after the tile's first column (always, in
    // a chunk without a reset), every entry is kept: one wave-wide test and a uniform
    // branch instead of a compare and a select per entry
    if (ti > tj && __builtin_amdgcn_ballot_w64(rho >= 16 * tj) == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            av[e] = -br * ex[e] * kk[e];
            pv[e] = scale * ex[e] * qk[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = 16 * tj + 4 * lg + e;
            const bool below = ti > tj;
            const float gam = ((below || c <= rr) && rho <= c) ? ex[e] : 0.f;
            av[e] = (below || c < rr) ? -br * gam * kk[e] : 0.f;
            pv[e] = scale * gam * qk[e];
        }
    }
    if constexpr (P::kBF16) {
        const int eo = dt_index(ti, tj >> 1) * 1024 + 16 * lane + 8 * (tj & 1);
        *reinterpret_cast<u32x2 *>(buf + L::oA + eo) = u32x2{pk_h(av[0], av[1]), pk_h(av[2], av[3])};
        if constexpr (WITH_O)
            *reinterpret_cast<u32x2 *>(buf + L::oPh + eo) = u32x2{pk_h(pv[0], pv[1]), pk_h(pv[2], pv[3])};
    } else {
        const int eo = tri_index(ti, tj) * 256 + 4 * lane;
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(buf + L::oA) + eo) = av;
        if constexpr (WITH_O) *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(buf + L::oPh) + eo) = pv;
    }
    return av;
}

// 16x16x16 product on the matrix cores with bf16 (fp32 for fp32 inputs) operands and
// fp32 accumulation:
// D = C + X Y for X in the A-operand layout (lane l: row l%16, columns 4 (l/16) + i) and
// Y in the accumulator layout (lane l: rows 4 (l/16) + i, column l%16); D comes out in the
// accumulator layout.  Read the other way round, mm16(C, Y, X) gives C + X Y in the
// A-operand layout.
__device__ __forceinline__ h16x4 pk4(f32x4 x) {
    return __builtin_bit_cast(h16x4, u32x2{pk_h(x[0], x[1]), pk_h(x[2], x[3])});
}
template <bool BF16>
__device__ __forceinline__ f32x4 mm16(f32x4 c, f32x4 x, f32x4 y) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(pk4(x), pk4(y), c, 0, 0, 0);
    } else {   // fp32 operands for fp32 inputs (four 16x16x4 steps)
#pragma unroll
        for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(x[j], y[j], c, 0, 0, 0);
        return c;
    }
}

// T_bb - I for one 16x16 block from N = -A_bb (strictly lower) in the A-operand layout.
// With D the 4x4 diagonal blocks of N and E the rest (strictly block-lower),
//     I - N = (I - G)(I - D),   G = E (I - D)^{-1},
// and D, G are both nilpotent of order 4 (D: 4x4 strictly lower blocks; G: strictly
// block-lower over four 4-row blocks), so
//     T = (I + A)^{-1} = (I - D)^{-1} (I - G)^{-1} = (I + D + D^2 + D^3)(I + G + G^2 + G^3),
// nine 16x16x16 products on the matrix cores, formed in registers (fp16 operands for
// bf16 inputs, fp32 for fp32 inputs).  Every intermediate stays O(1) for any keys: a
// truncated Neumann series over the whole 16x16 block, (I + N)(I + N^2)(I + N^4)(I + N^8),
// is exact too, but its terms grow like binomial coefficients when keys are correlated
// (|N^4| ~ 15 at a mean key cosine of 0.9, thousands for a repeated key), and fp16
// operands then lose the result to cancellation.  Stored in fragment order (lane l: row
// l%16, columns 4 (l/16) .. +3, at 4 l).
template <class E>
__device__ __forceinline__ void diag_inverse(f32x4 Nr, E *Tt, int lane) {
    constexpr bool BF = sizeof(E) == 2;
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 I4;
#pragma unroll
    for (int i = 0; i < 4; ++i) I4[i] = (4 * lg + i == lr) ? 1.f : 0.f;   // I, either layout
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // a lane's four A-layout entries are one 4-column group: the diagonal block of its
    // row exactly when that group is the row's
    const bool dblk = lg == (lr >> 2);
    const f32x4 Dr = dblk ? Nr : zero, Er = dblk ? zero : Nr;
    const f32x4 Dc = mm16<BF>(zero, Dr, I4);          // D, accumulator layout
    const f32x4 D2c = mm16<BF>(zero, Dr, Dc);
    const f32x4 D3c = mm16<BF>(zero, Dr, D2c);
    const f32x4 Dic = I4 + Dc + D2c + D3c;            // (I - D)^{-1}, accumulator layout
    const f32x4 Gc = mm16<BF>(zero, Er, Dic);         // G
    const f32x4 Gr = mm16<BF>(zero, Dic, Er);         // G, A-operand layout
    const f32x4 G2c = mm16<BF>(zero, Gr, Gc);
    const f32x4 G3c = mm16<BF>(zero, Gr, G2c);
    const f32x4 Gi1c = Gc + G2c + G3c;                // (I - G)^{-1} - I
    const f32x4 Dir = mm16<BF>(zero, Dic, I4);        // (I - D)^{-1}, A-operand layout
    // T - I = ((I - D)^{-1} - I) + (I - D)^{-1} ((I - G)^{-1} - I)
    const f32x4 Tm = mm16<BF>(Dir - I4, Gi1c, Dir);
    E *row = Tt + 4 * lane;
    if constexpr (sizeof(E) == 2) {
        *reinterpret_cast<u32x2 *>(row) = u32x2{pk_h(Tm[0], Tm[1]), pk_h(Tm[2], Tm[3])};
    } else {
        *reinterpret_cast<f32x4 *>(row) = Tm;
    }
}

// The Gram tiles of prep wave PW: waves 0..3 own diagonal block PW (formed, then inverted
// in registers); waves 4..6 two off-diagonal tiles each; wave 7 none (it owns the gates).
//   wave 4: (1,0) (2,0)   wave 5: (2,1) (3,0)   wave 6: (3,1) (3,2)
// In a column-slice workgroup, whose state waves without columns would only wait, three
// of them form the second tiles of waves 4..6 instead (NT1 = 1 there; see help_tile).
// Software-pipelined: the next tile's fragments are in flight while the current one is
// finished.  The stages are kept in order with scheduling barriers; the inverse's
// products are also kept apart from the Gram products (interleaving the two in one
// schedule gave wrong results).
template <int PW, int DK, class P, bool WITH_O, class L, int NT1 = 2>
__device__ __forceinline__ void prep_tiles(char *buf, const char *lds, uint32_t bo, int lane, float scale) {
    typedef typename P::E E;
    constexpr int KBK = DK / P::KB;
    constexpr int NT = PW < 4 ? 1 : PW < 7 ? NT1 : 0;
    constexpr int TI[2] = {PW < 4 ? PW : PW == 4 ? 1 : PW == 5 ? 2 : 3, PW == 4 ? 2 : 3};
    constexpr int TJ[2] = {PW < 4 ? PW : PW == 4 ? 0 : PW == 5 ? 1 : 1, PW == 4 ? 0 : PW == 5 ? 0 : 2};
    // fp32 fragments at d_k = 128 fill 96 registers per tile, more than fit next to the
    // prefetched next chunk: there each tile is loaded and multiplied in two halves of d_k
    constexpr bool PIPE = !(sizeof(E) == 4 && DK == 128);
    if constexpr (NT > 0 && !PIPE) {
        TileIn<P, KBK> in;
        f32x4 kk, qk, Nr;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            __builtin_amdgcn_sched_barrier(0);
            tile_load<DK, P, WITH_O, L, 0, KBK / 2>(in, buf, lds, bo, TI[n], TJ[n], lane);
            tile_mma<DK, P, WITH_O, 0, KBK / 2>(in, kk, qk);
            __builtin_amdgcn_sched_barrier(0);
            tile_load<DK, P, WITH_O, L, KBK / 2, KBK>(in, buf, lds, bo, TI[n], TJ[n], lane);
            tile_mma<DK, P, WITH_O, KBK / 2, KBK>(in, kk, qk);
            __builtin_amdgcn_sched_barrier(0);
            const f32x4 av = tile_store<DK, P, WITH_O, L>(buf, in.hr, in.lr, in.br, in.rho, in.hc, in.lc, kk, qk,
                                                          TI[n], TJ[n], lane, scale);
            if (n == 0) Nr = av;
        }
        if constexpr (PW < 4) {
            __builtin_amdgcn_sched_barrier(0);
            diag_inverse<E>(Nr, reinterpret_cast<E *>(buf + L::oT) + PW * 256, lane);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (NT > 0) {
        TileIn<P, KBK> in;
        f32x4 kk, qk, Nr;
        tile_load<DK, P, WITH_O, L>(in, buf, lds, bo, TI[0], TJ[0], lane);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            __builtin_amdgcn_sched_barrier(0);
            tile_mma<DK, P, WITH_O>(in, kk, qk);
            const float hr = in.hr, lr = in.lr, br = in.br;
            const int rho = in.rho;
            const f32x4 hc = in.hc, lc = in.lc;
            __builtin_amdgcn_sched_barrier(0);
            if (n + 1 < NT) tile_load<DK, P, WITH_O, L>(in, buf, lds, bo, TI[n + 1], TJ[n + 1], lane);
            __builtin_amdgcn_sched_barrier(0);
            const f32x4 av = tile_store<DK, P, WITH_O, L>(buf, hr, lr, br, rho, hc, lc, kk, qk, TI[n], TJ[n],
                                                          lane, scale);
            if (n == 0) Nr = av;
        }
        if constexpr (PW < 4) {
            __builtin_amdgcn_sched_barrier(0);
            diag_inverse<E>(Nr, reinterpret_cast<E *>(buf + L::oT) + PW * 256, lane);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// One off-diagonal Gram tile (TI > TJ) formed by a helper wave: the second tile of prep
// wave 4, 5 or 6 (HW = 0, 1, 2), the same arithmetic as there.
template <int HW, int DK, class P, bool WITH_O, class L>
__device__ __forceinline__ void help_tile(char *buf, const char *lds, uint32_t bo, int lane, float scale) {
    typedef typename P::E E;
    constexpr int KBK = DK / P::KB;
    constexpr int TI = HW == 2 ? 3 : HW + 2, TJ = HW == 2 ? 2 : 0;
    constexpr bool PIPE = !(sizeof(E) == 4 && DK == 128);
    TileIn<P, KBK> in;
    f32x4 kk, qk;
    if constexpr (PIPE) {
        tile_load<DK, P, WITH_O, L>(in, buf, lds, bo, TI, TJ, lane);
        tile_mma<DK, P, WITH_O>(in, kk, qk);
    } else {
        tile_load<DK, P, WITH_O, L, 0, KBK / 2>(in, buf, lds, bo, TI, TJ, lane);
        tile_mma<DK, P, WITH_O, 0, KBK / 2>(in, kk, qk);
        __builtin_amdgcn_sched_barrier(0);
        tile_load<DK, P, WITH_O, L, KBK / 2, KBK>(in, buf, lds, bo, TI, TJ, lane);
        tile_mma<DK, P, WITH_O, KBK / 2, KBK>(in, kk, qk);
    }
    __builtin_amdgcn_sched_barrier(0);
    tile_store<DK, P, WITH_O, L>(buf, in.hr, in.lr, in.br, in.rho, in.hc, in.lc, kk, qk, TI, TJ, lane, scale);
}

// ---------------------------------------------------------------- kernel
// HELP: every block is a column slice in which at least three state waves have no columns
// (the launcher guarantees it); those form three of the Gram tiles (help_tile).
// MP: every sequence has 2 h_v head units: the first h_v the usual ones, the second h_v
// the same chains with V taken as zero and S started from the identity (d_k = d_v), so
// that their final S is the window's transition map M (S_end = M S_start + S_local);
// their states follow the first n_seqs h_v ones in S_out, stored as 16 x 16 tiles (tile
// (i, j) of a map at 256 (i d/16 + j) floats, row-major inside) for the combine's loads.
template <int DK, int DV, int W, class P, bool WITH_O, bool HELP, bool MP = false>
__global__ void __launch_bounds__(64 * (W / 16 + NPW)) gdn_chunk_ws_kernel(ChunkArgs a)
{
    constexpr int NSW = W / 16;            // state waves: one 16-column tile of S each
    constexpr int NTHR = 64 * (NSW + NPW);
    typedef typename P::E E;
    typedef typename P::Frag Frag;
    typedef Lds<DK, W, P, WITH_O> L;
    constexpr int RT = DK / 16;            // row tiles of S
    constexpr int KBK = DK / P::KB;        // k-blocks over d_k
    constexpr int KBT = CH / P::KB;        // k-blocks over the chunk's tokens
    constexpr int NCB = DV / W;            // column blocks per head
    constexpr int RBK = L::RBK;
    static_assert(L::bytes <= 160 * 1024, "LDS plan");
    static_assert(!MP || (DK == DV && !WITH_O), "transition maps: square states, no outputs");
    // a chunk buffer's offset leaves the bits that the fragment XORs touch alone
    static_assert(L::BUF % L::RBK == 0 && L::BUF % L::RBV == 0 && L::BUF % 256 == 0, "buffer alignment");

    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    int64_t *gMisc = reinterpret_cast<int64_t *>(smem + L::oMisc);
    int *pctr = reinterpret_cast<int *>(smem + L::oMisc + 8);
    int *pfail = reinterpret_cast<int *>(smem + L::oMisc + 12);
    int *qctr = reinterpret_cast<int *>(smem + L::oMisc + 16);   // Q rows released (single Q buffer)

    const int tid = threadIdx.x, lane0 = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int lane = lane0, lr = lane & 15, lg = lane >> 4;
    const bool is_state = wave < NSW;

    // ---- block -> work unit (sequence, v-head, column block) and its column slice.
    // Blocks [0, n_full) take whole units.  The units that would leave the last round
    // of the grid partly empty are instead split by columns into 2^split slices, one
    // block each (the columns of S evolve independently; each slice repeats the
    // unit's prep work), so that round fills more of the chip.  Within each range the
    // order is XCD-aware: consecutive logical blocks (the slices of a unit, the v-heads
    // of one q/k head, the heads of one sequence) share an XCD's L2.
    //
    // Packed sequences of different lengths (2 to kOrderSeqs of them) are taken longest
    // window first: every block ranks the sequences by chunk count (ties by index) in LDS
    // and maps its logical position through that order, so that the long chains start in
    // the first round and the short ones fill in behind them.  Whole units then go out in
    // groups of 16 blocks, the two v-heads of a q/k-head pair on one XCD (blocks 2x and
    // 2x + 1 of a group to XCD x).  Equal lengths keep the interleave above.
    const int64_t nblk = (int64_t)gridDim.x;
    const int hvu = MP ? 2 * a.h_v : a.h_v;        // head units per sequence
    const int64_t ups = (int64_t)NCB * hvu;        // units per sequence
    int64_t unit;
    int slice = 0;
    int ncols = W;                         // columns of this block
    // (the ordering pass keeps every sequence's cu_seqlens pair and r in LDS, so that the
    // window below comes from there instead of from a second round of global loads)
    const int *lcu0 = nullptr, *lcu1 = nullptr, *lrr = nullptr;
    {
        bool lpt = false;
        const int *lord = nullptr;
        if (a.n_seqs >= 2 && a.n_seqs <= kOrderSeqs) {
            // (buffer 1's K rows are free until the first chunk is staged)
            int *lb0 = reinterpret_cast<int *>(smem + L::BUF + L::oK);
            int *lb1 = lb0 + kOrderSeqs, *lr = lb1 + kOrderSeqs;
            int *lnch = lr + kOrderSeqs;
            int *lo = lnch + kOrderSeqs;
            int *ldiff = lo + kOrderSeqs;
            if (tid == 0) *ldiff = 0;
            for (int m = tid; m < a.n_seqs; m += NTHR) {
                const int b0 = a.cu[m], b1 = a.cu[m + 1];
                const int rr = a.r ? a.r[m] : 0;
                lb0[m] = b0;
                lb1[m] = b1;
                lr[m] = rr;
                int64_t len = a.r ? (int64_t)rr : (int64_t)b1 - b0;
                if (b0 < 0 || b1 < b0 || b1 > a.total_tokens || len < 0 || len > (int64_t)b1 - b0) len = 0;
                lnch[m] = (int)((len + CH - 1) / CH);
            }
            __syncthreads();
            for (int m = tid; m < a.n_seqs; m += NTHR) {
                const int km = lnch[m];
                int rank = 0;
                for (int j = 0; j < a.n_seqs; ++j) {
                    const int kj = lnch[j];
                    rank += (kj > km || (kj == km && j < m)) ? 1 : 0;
                }
                lo[rank] = m;
                if (km != lnch[0]) *ldiff = 1;
            }
            __syncthreads();
            lpt = *ldiff != 0;
            lord = lo;
            lcu0 = lb0;
            lcu1 = lb1;
            lrr = lr;
        }
        int64_t b = blockIdx.x;
        if (b < a.n_full) {
            if (lpt) {
                if (b < (a.n_full & ~(int64_t)15))
                    b = (b & ~(int64_t)15) + 2 * (b & 7) + ((b >> 3) & 1);
                unit = (int64_t)lord[b / ups] * ups + b % ups;
            } else {
                if ((a.n_full & 7) == 0) b = (b & 7) * (a.n_full >> 3) + (b >> 3);
                unit = b;
            }
        } else {
            const int64_t m = nblk - a.n_full;
            b -= a.n_full;
            if ((m & 7) == 0) b = (b & 7) * (m >> 3) + (b >> 3);
            unit = a.n_full + (b >> a.split);
            if (lpt) unit = (int64_t)lord[unit / ups] * ups + unit % ups;
            slice = (int)(b & ((1 << a.split) - 1));
            ncols = W >> a.split;
        }
        // the unit is the same in every lane: scalar registers, scalar address arithmetic
        unit = uniform64(unit);
    }
    // (the 64-bit divisions expand to vector code: their results go back to scalar registers)
    const int cb = __builtin_amdgcn_readfirstlane((int)(unit % NCB));
    const int hh = __builtin_amdgcn_readfirstlane((int)((unit / NCB) % hvu));
    const int n = __builtin_amdgcn_readfirstlane((int)(unit / ups));
    const bool mp = MP && hh >= a.h_v;                  // a transition-map unit
    const int h = mp ? hh - a.h_v : hh;
    const int c_lo = cb * W + slice * ncols;            // first d_v column of the block
    const int nact = ncols / 16;                        // state waves with columns
    const int hk = __builtin_amdgcn_readfirstlane((int)(((int64_t)h * a.h_qk) / a.h_v));
    const bool replay = a.r != nullptr;

    // ---- window selection (validates the device-resident cu_seqlens / r)
    if (blockIdx.x == 0) {
        int bad = 0;
        for (int m = tid; m < a.n_seqs; m += NTHR) {
            const int64_t b0 = a.cu[m], b1 = a.cu[m + 1];
            if (b0 < 0 || b1 < b0 || b1 > a.total_tokens) bad = 1;
            if (replay && (a.r[m] < 0 || a.r[m] > b1 - b0)) bad = 1;
        }
        if (WITH_O && replay && wave == 0) {   // the packed outputs must fit o_out
            int64_t tot = 0;
            for (int m = lane; m < a.n_seqs; m += 64) tot += a.r[m];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
            if (tot > a.total_out) bad = 1;
        }
        bad = __syncthreads_or(bad);
        if (tid == 0 && bad) atomicOr(a.status, kStatusBitInput);
    }
    const int64_t beg = __builtin_amdgcn_readfirstlane(lcu0 ? lcu0[n] : a.cu[n]);
    const int64_t end = __builtin_amdgcn_readfirstlane(lcu1 ? lcu1[n] : a.cu[n + 1]);
    if (beg < 0 || end < beg || end > a.total_tokens) return;
    const int64_t rn = replay ? (int64_t)__builtin_amdgcn_readfirstlane(lrr ? lrr[n] : a.r[n]) : end - beg;
    if (rn < 0 || rn > end - beg) return;
    const int64_t wbeg = end - rn;              // first token of the window
    if (wave == 0) {
        int64_t row0 = beg;
        if (replay) {
            int64_t s = 0;
            for (int m = lane; m < n; m += 64) s += lrr ? lrr[m] : a.r[m];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
            row0 = s;
        }
        if (lane == 0) {
            gMisc[0] = row0;
            *pctr = 0;
            *pfail = 0;
            *qctr = 0;
        }
    }
    if constexpr (P::kBF16) {   // the tile pairs' upper halves are zero and never written
        for (int i = 16 * tid; i < L::BUF - L::oA; i += 16 * NTHR) {
            *reinterpret_cast<u32x4 *>(smem + L::oA + i) = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(smem + L::BUF + L::oA + i) = u32x4{0u, 0u, 0u, 0u};
        }
    }
    __syncthreads();
    const int64_t orow0 = gMisc[0];
    // output rows (and cu_out) must fit; without outputs only cu_out uses them
    if (orow0 < 0 || orow0 + rn > ((replay && WITH_O) ? a.total_out : a.total_tokens)) return;
    if (a.cu_out && !mp && h == 0 && c_lo == 0 && tid == 0) {
        a.cu_out[n] = (int32_t)orow0;
        if (n == a.n_seqs - 1) a.cu_out[n + 1] = (int32_t)(orow0 + rn);
    }
    const int64_t nch = (rn + CH - 1) / CH;

    const E *qg = reinterpret_cast<const E *>(a.q);
    const E *kg = reinterpret_cast<const E *>(a.k);
    const E *vg = reinterpret_cast<const E *>(a.v);
    const int64_t sbase = uniform64((((int64_t)(mp ? a.n_seqs : 0) + n) * a.h_v + h) * DK * DV);

    // HELP: three state waves without columns form the second Gram tiles of prep waves
    // 4..6, which shortens the prep waves' chain (it sets the chunk period when only a few
    // state waves have columns)
    if (is_state && wave >= nact) {
        const int hw = wave - nact;
        if (HELP && hw < 3) {
            int htarget = 0;
            auto help = [&](int64_t cc) {
                const int lane = fresh_lane();
                htarget += NPW;                     // after the prep waves' staging of chunk cc
                lds_wait_ge(pctr, htarget, pfail);
                const uint32_t bo = (uint32_t)((cc & 1) * L::BUF);
                char *buf = smem + bo;
                switch (hw) {
                case 0: help_tile<0, DK, P, WITH_O, L>(buf, smem, bo, lane, a.scale); break;
                case 1: help_tile<1, DK, P, WITH_O, L>(buf, smem, bo, lane, a.scale); break;
                default: help_tile<2, DK, P, WITH_O, L>(buf, smem, bo, lane, a.scale); break;
                }
            };
            if (nch > 0) help(0);
            sync_lds();                              // chunk 0 prepared
            for (int64_t c = 0; c < nch; ++c) {
                if (c + 1 < nch) help(c + 1);
                sync_lds();
            }
        } else {
            // a state wave without columns (a split block): only the state waves' barriers
            sync_lds();
            for (int64_t c = 0; c < nch; ++c) sync_lds();
        }
    } else if (is_state) {
        // =====================================================================
        // state waves
        const int col0 = c_lo + wave * 16;         // first d_v column of this wave
        f32x4 S[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (mp) {                                // a transition map starts at the identity
#pragma unroll
                for (int i = 0; i < 4; ++i) S[rt][i] = (16 * rt + 4 * lg + i == col0 + lr) ? 1.f : 0.f;
            } else if (a.S0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[rt][i] = a.S0[sbase + (int64_t)(16 * rt + 4 * lg + i) * DV + col0 + lr];
            } else {
                S[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        // fp32 inputs: V rows of a chunk in accumulator layout, from global memory (rows
        // past the window read as 0; a chunk past the window gets an empty buffer and
        // touches no memory).  bf16 inputs take V from the chunk buffer instead.
        const int vct = (c_lo - cb * W) / 16 + wave;   // 16-column tile of the staged V rows
        const uint32_t vrow = (uint32_t)a.h_v * (uint32_t)(DV * sizeof(E));   // bytes per token
        typename Raw<P>::T vreg[4][4];
        auto fetch_v = [&](int64_t cc) {
            const int lane = fresh_lane();
            const int64_t ln = (rn - cc) < CH ? (rn - cc) : CH;
            // (a transition map reads V as zero: an empty buffer, every load returns 0)
            const Rsrc rs = make_rsrc(vg + ((wbeg + cc) * a.h_v + h) * (int64_t)DV + col0,
                                      mp ? 0 : ln * (int64_t)vrow);
            // token rows 16 tt + 4 (lane/16) + i: one running offset, one add per load
            uint32_t vo = (uint32_t)(4 * (lane >> 4)) * vrow + (uint32_t)(lane & 15) * (uint32_t)sizeof(E);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vreg[tt][i] = load_e<P>(rs, vo);
                    vo += (i == 3 ? 13u : 1u) * vrow;
                    asm volatile("" : "+v"(vo));   // kept as a chain, not re-derived per load
                }
        };
        // the initial state is in registers before the loop, so no wait for it is left
        // inside the loop (vmcnt(0) only; expcnt and lgkmcnt at their maxima)
        __builtin_amdgcn_s_waitcnt(0x0F70);
        if constexpr (!P::kBF16) {
            if (nch > 0) fetch_v(0);
        }
        sync_lds();                                  // chunk 0 prepared

        for (int64_t c = 0; c < nch; ++c) {
            const int64_t c0 = c * CH;
            const int len = (int)((rn - c0) < CH ? (rn - c0) : CH);
            // lane-derived indices are recomputed each chunk instead of being held in
            // registers across the whole loop
            const int lane = fresh_lane();
            const int lr = lane & 15, lg = lane >> 4;
            const char *buf = smem + (c & 1) * L::BUF;
            const char *Ks = buf + L::oK;
            const char *Qs = L::q_rows(smem, buf);
            const float *gH = reinterpret_cast<const float *>(buf + L::oGate);
            const float *gE = gH + CH, *gB = gE + CH, *gL = gB + CH, *gEs = gL + CH;
            // fragment address offsets, the chunk buffer's folded in (frag_off, tr_off)
            const uint32_t bo = (uint32_t)((c & 1) * L::BUF);
            const uint32_t fo = frag_off<RBK>(lane);
            const uint32_t fob = fo + bo, qob = L::Q1 ? fo : fob;
            const char *Qb = smem + (L::Q1 ? L::oQ1 : L::oQ);

            // X = K S and (Q S)^T = S^T Q^T, by k-block (S rounded once to the operand type)
            f32x4 X[4], OT[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                X[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
                OT[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int kb = 0; kb < KBK; ++kb) {
                Frag sh;
                if constexpr (P::kBF16) sh = bfrag(S[2 * kb], S[2 * kb + 1]);
                else sh = S[kb];
                // this k-block's offsets formed here, not all four ahead of time
                uint32_t fk = fob;
                asm volatile("" : "+v"(fk));
                fk ^= 64u * kb;
                const uint32_t qk = L::Q1 ? (qob ^ (64u * kb)) : fk;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    X[tt] = mma(X[tt], frag_at<Frag>(smem + L::oK + 16 * tt * RBK + fk), sh);
                    if constexpr (WITH_O) {
                        const Frag qf = frag_at<Frag>(Qb + 16 * tt * RBK + qk);
                        OT[tt] = mma(OT[tt], sh, qf);
                    }
                }
            }
            if constexpr (L::Q1) {   // this chunk's Q rows are read: they may be refilled
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
                if (lane == 0) __hip_atomic_fetch_add(qctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            // Y = b (V - e X), in place
            const uint32_t vo = P::kBF16 ? ((tr_off<L::RBV>(lane) + bo) ^ (uint32_t)(64 * (vct >> 1))) + 8u * (vct & 1)
                                         : 0u;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const f32x4 br = *reinterpret_cast<const f32x4 *>(gB + 16 * tt + 4 * lg);
                const f32x4 er = *reinterpret_cast<const f32x4 *>(gE + 16 * tt + 4 * lg);
                f32x4 vv;
                if constexpr (P::kBF16) {
                    const u32x2 w = frag_v_at<L::RBV>(smem + L::oV, vo, tt);
                    vv = f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                                __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) vv[i] = v_at<P>(vreg[tt][i]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) X[tt][i] = br[i] * (vv[i] - er[i] * X[tt][i]);
            }
            // fp32 inputs: the next chunk's V lands while this one is processed
            if constexpr (!P::kBF16) fetch_v(c0 + CH);

            // (I + A) U = Y by 16-row block forward substitution
            f32x4 U[4];
            if constexpr (P::kBF16) {
                const char *Ad = buf + L::oA;
                const uint16_t *Tt = reinterpret_cast<const uint16_t *>(buf + L::oT);
                // tiles (b, j < b): a 16x32 pair, or a 16x16 product when only tile (1, 0)
                // exists.  A 16x16x16 product only ever accumulates onto values a vector
                // instruction has read or written since the last matrix product (X after Y,
                // z after its conversion to bf16): a 16x16x16 product that accumulates
                // directly onto a 16x16x32 result gave wrong results, so (3, 2) stays a
                // zero-padded 16x32 product in the 16x32 chain.
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    f32x4 z = X[b];
                    if (b == 1) z = mma16(z, frag_dt_first(Ad, dt_index(1, 0), lane), bfrag16(U[0]));
                    if (b >= 2) z = mma(z, frag_dt(Ad, dt_index(b, 0), lane), bfrag(U[0], U[1]));
                    if (b == 3) z = mma(z, frag_dt(Ad, dt_index(3, 1), lane), bfrag(U[2], zero));
                    U[b] = mma16(z, frag_t16(Tt, b, lane), bfrag16(z));
                }
            } else {
                const float *At = reinterpret_cast<const float *>(buf + L::oA);
                const float *Tt = reinterpret_cast<const float *>(buf + L::oT);
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    f32x4 z = X[b];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (j < b) z = mma(z, frag_tile(At, tri_index(b, j), lane), U[j]);
                    U[b] = mma(z, frag_tile(Tt, b, lane), z);
                }
            }

            // O^T = (S^T Q^T) diag(scale e) + U^T P^T; lane: token 16 tt + l%16, d_v
            // columns col0 + 4 (l/16) + i
            if constexpr (WITH_O) {
                Frag uh[KBT];
#pragma unroll
                for (int kb = 0; kb < KBT; ++kb) {
                    if constexpr (P::kBF16) uh[kb] = bfrag(U[2 * kb], U[2 * kb + 1]);
                    else uh[kb] = U[kb];
                }
                const char *Ph = buf + L::oPh;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    OT[tt] *= gEs[16 * tt + lr];
#pragma unroll
                    for (int kb = 0; kb < KBT; ++kb) {
                        if (kb * P::KB < 16 * tt + 16) {
                            if constexpr (P::kBF16) {
                                OT[tt] = mma(OT[tt], uh[kb], frag_dt(Ph, dt_index(tt, kb), lane));
                            } else {
                                OT[tt] = mma(OT[tt], uh[kb],
                                             frag_tile(reinterpret_cast<const float *>(Ph), tri_index(tt, kb), lane));
                            }
                        }
                    }
                }
                {   // (the launcher instantiates WITH_O only for a non-null o_out)
                    // rows past the window end fall outside the buffer and are dropped
                    const int64_t orow_first = replay ? orow0 + c0 : wbeg + c0;
                    const bool f32o = !P::kBF16 || a.o_f32;
                    const uint32_t osz = f32o ? 4u : 2u;
                    const uint32_t orow = (uint32_t)a.h_v * (uint32_t)DV * osz;
                    const Rsrc rs = make_rsrc(reinterpret_cast<const char *>(a.o_out) +
                                                  ((orow_first * a.h_v + h) * DV + col0) * (int64_t)osz,
                                              (int64_t)len * orow);
                    const uint32_t ob = (uint32_t)lr * orow + (uint32_t)(4 * lg) * osz;
                    if (f32o) {
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt)
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, OT[tt]), rs,
                                                                   ob + (uint32_t)(16 * tt) * orow, 0, 0);
                    } else {
                        // two token tiles per store: swapping lane rows 1, 3 of tile ta with rows
                        // 0, 2 of tile tb gives every lane 8 consecutive columns (16 bytes) of one
                        // token -- rows 0, 2 token 16 ta + l%16, rows 1, 3 token 16 tb + l%16
#pragma unroll
                        for (int tp = 0; tp < 2; ++tp) {
                            const int ta = 2 * tp, tb = 2 * tp + 1;
                            const auto s0 = __builtin_amdgcn_permlane16_swap(pk_bf16(OT[ta][0], OT[ta][1]),
                                                                             pk_bf16(OT[tb][0], OT[tb][1]), false, false);
                            const auto s1 = __builtin_amdgcn_permlane16_swap(pk_bf16(OT[ta][2], OT[ta][3]),
                                                                             pk_bf16(OT[tb][2], OT[tb][3]), false, false);
                            const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
                            const uint32_t tok = (uint32_t)(16 * ((lg & 1) ? tb : ta) + lr);
                            __builtin_amdgcn_raw_buffer_store_b128(w, rs, tok * orow + (uint32_t)(16 * (lg >> 1)), 0, 0);
                        }
                    }
                }
            }

            // S <- e_last S + K^T diag(G_last) U, on the stored state S~ = S / sig: the
            // gate rows carry e sig_{c-1} and G_last / sig_c, so the decay costs nothing
            // here except on the rare chunks that renormalise S~ (factor != 1)
            {
                const float rn = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(gH[6 * CH])));
                if (rn != 1.f) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) S[rt] *= rn;
                }
                Frag dh[KBT];
                const uint32_t tob = tr_off<RBK>(lane) + bo;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const f32x4 l4 = *reinterpret_cast<const f32x4 *>(gL + 16 * tt + 4 * lg);
#pragma unroll
                    for (int i = 0; i < 4; ++i) U[tt][i] *= l4[i];
                }
#pragma unroll
                for (int kb = 0; kb < KBT; ++kb) {
                    if constexpr (P::kBF16) dh[kb] = bfrag(U[2 * kb], U[2 * kb + 1]);
                    else dh[kb] = U[kb];
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    f32x4 s = S[rt];
#pragma unroll
                    for (int kb = 0; kb < KBT; ++kb) {
                        if constexpr (P::kBF16) {
                            s = mma(s, frag_kt_at<RBK>(smem + L::oK, tob, rt, kb), dh[kb]);
                        } else {
                            s = mma(s, frag_cols_f32<RBK>(Ks, 16 * rt, kb, lane), dh[kb]);
                        }
                    }
                    S[rt] = s;
                }
            }
            sync_lds();   // this chunk's buffer is free; the next one is prepared
        }

        // ---- state write-back: S = sig S~, sig from the last chunk's gate rows (lane
        // indices derived afresh, so that no address stays live across the chunk loop)
        const float sig = nch > 0 ? reinterpret_cast<const float *>(smem + ((nch - 1) & 1) * L::BUF +
                                                                    L::oGate)[6 * CH + 1]
                                  : 1.f;
        const int wl = fresh_lane();
        if (mp) {   // a transition map: 16 x 16 tiles, each 1 KB contiguous and row-major inside
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a.S_out[sbase + (int64_t)(rt * (DV / 16) + col0 / 16) * 256 + (4 * (wl >> 4) + i) * 16 + (wl & 15)] =
                        S[rt][i] * sig;
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a.S_out[sbase + (int64_t)(16 * rt + 4 * (wl >> 4) + i) * DV + col0 + (wl & 15)] = S[rt][i] * sig;
        }
    } else {
        // =====================================================================
        // prep waves: chunk c + 1's operands while the state waves process chunk c
        const int pw = wave - NSW;                 // 0..NPW-1
        int target = 0;
        // K / Q staging: a thread moves "units" of a row; a bf16 unit is the two 16-byte
        // vectors (columns 32b + 8q .. +7 and 32b + 16 + 8q .. +7) that make up logical
        // chunks 4b + 2q and 4b + 2q + 1, an fp32 unit one vector (one chunk)
        constexpr int VPU = P::kBF16 ? 2 : 1;                 // vectors per unit
        constexpr int NPU = P::kBF16 ? DK / 16 : RBK / 16;    // units per row
        constexpr int UT = CH * NPU;                          // units per matrix
        constexpr int TH = 64 * NPW;                          // prep threads
        constexpr int RPJ = TH / NPU;                         // rows per round
        constexpr int NR = (UT + TH - 1) / TH;                // rounds per chunk
        static_assert(TH % NPU == 0 && (UT <= TH || UT % TH == 0), "unit map");
        const uint32_t krow = (uint32_t)a.h_qk * (uint32_t)RBK;    // bytes per token
        const uint32_t grow = (uint32_t)a.h_v * 4u;
        u32x4 kpf[NR * VPU], qpf[NR * VPU];
        uint32_t gpf = 0, bpf = 0;
        Gates gt = {0.f, 0.f, 0.f, 0.f, 0.f, -1};
        float sig = 1.f;                           // scale of the stored state (gate wave)
        constexpr int GW = NPW - 1;                // the wave that owns the gates
        // this lane's staging unit, the same in every chunk: its offset in a chunk's K / Q
        // rows and its LDS slots (a bf16 unit is logical chunks c0 and c0 + 1 of a row; the
        // lanes of the upper half of a row write them in the other order, so that each
        // store's eight lanes of one row hit eight distinct 16-byte slots modulo 128 bytes,
        // the stores' bank rule).  The column-slice variant with helper waves keeps the plain
        // order: with one state wave per slice the LDS is lightly loaded, and the register
        // selects the swap costs sit on the preparation chain that paces such a slice
        // (measured: the 8K and slow-decay layers 1.4 and 2.1 % faster this way; without
        // the swap in every variant the stack was 0.3 % slower, so the whole-unit one keeps it)
        const int spt = 64 * pw + fresh_lane();
        const bool s_act = UT >= TH || spt < UT;   // with fewer units than threads, the last waves idle
        const int spu = spt % NPU, srow = spt / NPU;
        // V rows (bf16 inputs): the same kind of units over the block's columns, rounded out
        // to whole 32-column blocks, at their places in a W-column row; copied without
        // conversion (the state waves read them with transposing reads).  At most one unit
        // per thread.
        static_assert(CH * (W / 16) <= TH, "V unit map");
        constexpr bool STAGE_V = P::kBF16;
        const uint32_t vrowp = (uint32_t)a.h_v * (uint32_t)(DV * sizeof(E));   // bytes per token
        u32x4 vpf[2];
        const int nuv = (ncols < 32 ? 32 : ncols) / 16;          // units per row
        const int srowv = spt >> __builtin_ctz(nuv);
        const int spuv = 2 * ((c_lo - cb * W) >> 5) + (spt & (nuv - 1));
        const bool v_act = STAGE_V && srowv < CH;
        const uint32_t v_vo = (uint32_t)srowv * vrowp + (uint32_t)(64 * (spuv >> 1) + 16 * (spuv & 1));
        const bool v_sw = !HELP && (spuv & 4) != 0;
        int v_oa = 0, v_ob = 0;
        if constexpr (STAGE_V) {
            const int c0 = 4 * (spuv >> 1) + 2 * (spuv & 1);
            v_oa = chunk_at<L::RBV>(srowv, v_sw ? c0 + 1 : c0);
            v_ob = chunk_at<L::RBV>(srowv, v_sw ? c0 : c0 + 1);
        }
        const uint32_t s_vo = (uint32_t)srow * krow +
                              (uint32_t)(P::kBF16 ? 64 * (spu >> 1) + 16 * (spu & 1) : 16 * spu);
        const bool s_sw = P::kBF16 && !HELP && (spu & 4) != 0;
        int s_oa[NR], s_ob[NR];
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const int c0 = P::kBF16 ? 4 * (spu >> 1) + 2 * (spu & 1) : spu;
            s_oa[j] = chunk_at<RBK>(srow + RPJ * j, s_sw ? c0 + 1 : c0);
            s_ob[j] = chunk_at<RBK>(srow + RPJ * j, s_sw ? c0 : c0 + 1);
        }
        // the chunk starting at token cc of the window into registers (rows past the
        // window read as 0: g = b = 0 there; a chunk past the window reads nothing)
        auto fetch = [&](int64_t cc) {
            const int lane = fresh_lane();
            const int64_t ln = (rn - cc) < CH ? (rn - cc) : CH;
            const int64_t t0 = wbeg + cc;
            if (pw == GW) {   // first, so that waiting for them waits for nothing else
                const Rsrc rg = make_rsrc(a.g + t0 * a.h_v + h, ln * (int64_t)grow);
                const Rsrc rb = make_rsrc(a.beta + t0 * a.h_v + h, ln * (int64_t)grow);
                gpf = __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)lane * grow, 0, 0);
                bpf = __builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)lane * grow, 0, 0);
            }
            const int64_t koff = (t0 * a.h_qk + hk) * (int64_t)DK;
            const Rsrc rk = make_rsrc(kg + koff, ln * (int64_t)krow);
            const Rsrc rq = make_rsrc(qg + koff, ln * (int64_t)krow);
            if (s_act) {
#pragma unroll
                for (int j = 0; j < NR; ++j)
#pragma unroll
                    for (int v = 0; v < VPU; ++v) {
                        const uint32_t o = s_vo + (uint32_t)(RPJ * j) * krow + 32u * v;
                        kpf[VPU * j + v] = __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0);
                        if (WITH_O) qpf[VPU * j + v] = __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0);
                    }
            }
            if constexpr (STAGE_V) {
                if (v_act) {
                    // (a transition map stages V = 0: an empty buffer, every load returns 0)
                    const Rsrc rv = make_rsrc(vg + ((t0 * a.h_v + h) * (int64_t)DV + cb * W),
                                              mp ? 0 : ln * (int64_t)vrowp);
                    vpf[0] = __builtin_amdgcn_raw_buffer_load_b128(rv, v_vo, 0, 0);
                    vpf[1] = __builtin_amdgcn_raw_buffer_load_b128(rv, v_vo + 32u, 0, 0);
                }
            }
        };

        // prepare chunk cc into buffer cc & 1:
        //   step 1: K, Q, V (bf16 inputs; fetched one chunk earlier) and the gates
        //           (scanned one chunk earlier) into LDS; fetch chunk cc + 1
        //   step 2: after the prep waves' barrier, each wave's Gram tiles and diagonal
        //           inverse; the gate scan of chunk cc + 1 (wave GW)
        auto prep = [&](int64_t cc) {
            const int lane = fresh_lane();
            // step 1 is what every prep wave's barrier, and through it the state waves,
            // waits for: with all eight state waves busy it issues ahead of their work on the
            // same SIMD (measured: 6 % off the 36-layer replay; raising the Gram tiles as well
            // gains less); a column-slice block, with one or a few state waves, gains nothing
            // from it and loses up to 7 %, so it keeps the default priority
            if (nact == NSW) __builtin_amdgcn_s_setprio(3);
            const uint32_t bo = (uint32_t)((cc & 1) * L::BUF);
            char *buf = smem + bo;
            char *Ks = buf + L::oK;
            char *Qs = const_cast<char *>(L::q_rows(smem, buf));
            if (s_act) {
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    if constexpr (P::kBF16) {
                        const bool sw = s_sw;
                        const int oa = s_oa[j], ob = s_ob[j];
                        // bf16 in global memory, fp16 in LDS (the matrix operand type)
                        const u32x4 a0 = kpf[2 * j], a1 = kpf[2 * j + 1];
                        const u32x4 k0 = {bf2_to_h2(a0.x), bf2_to_h2(a0.y), bf2_to_h2(a1.x), bf2_to_h2(a1.y)};
                        const u32x4 k1 = {bf2_to_h2(a0.z), bf2_to_h2(a0.w), bf2_to_h2(a1.z), bf2_to_h2(a1.w)};
                        *reinterpret_cast<u32x4 *>(Ks + oa) = sw ? k1 : k0;
                        *reinterpret_cast<u32x4 *>(Ks + ob) = sw ? k0 : k1;
                        if (WITH_O) {
                            const u32x4 b0 = qpf[2 * j], b1 = qpf[2 * j + 1];
                            const u32x4 q0 = {bf2_to_h2(b0.x), bf2_to_h2(b0.y), bf2_to_h2(b1.x), bf2_to_h2(b1.y)};
                            const u32x4 q1 = {bf2_to_h2(b0.z), bf2_to_h2(b0.w), bf2_to_h2(b1.z), bf2_to_h2(b1.w)};
                            *reinterpret_cast<u32x4 *>(Qs + oa) = sw ? q1 : q0;
                            *reinterpret_cast<u32x4 *>(Qs + ob) = sw ? q0 : q1;
                        }
                    } else {
                        const int o = s_oa[j];
                        *reinterpret_cast<u32x4 *>(Ks + o) = kpf[j];
                        if (WITH_O && !L::Q1) *reinterpret_cast<u32x4 *>(Qs + o) = qpf[j];
                    }
                }
            }
            if constexpr (L::Q1) {
                // the single Q buffer still holds chunk cc - 1's rows until every state
                // wave with columns has finished its Q S products of that chunk
                lds_wait_ge(qctr, (int)cc * nact, pfail);
                if (s_act) {
#pragma unroll
                    for (int j = 0; j < NR; ++j) *reinterpret_cast<u32x4 *>(Qs + s_oa[j]) = qpf[j];
                }
            }
            if constexpr (STAGE_V) {
                if (v_act) {
                    char *Vs = buf + L::oV;
                    const u32x4 a0 = vpf[0], a1 = vpf[1];
                    const u32x4 v0 = {a0.x, a0.y, a1.x, a1.y}, v1 = {a0.z, a0.w, a1.z, a1.w};
                    *reinterpret_cast<u32x4 *>(Vs + v_oa) = v_sw ? v1 : v0;
                    *reinterpret_cast<u32x4 *>(Vs + v_ob) = v_sw ? v0 : v1;
                }
            }
            if (pw == GW) {
                // the state waves keep S~ = S / sig: the chunk's decay e_last goes into sig,
                // and into S~ (factor rn) only when sig would drop below kSigMin or the
                // chunk holds a reset (e_last = 0); then sig restarts at 1.  fp16 operands
                // (the bf16 path) keep |S~| <= 64 |S| that way; fp32 ones only need range.
                constexpr float kSigMin = P::kBF16 ? 0x1p-6f : 0x1p-60f;
                const float el = __shfl(gt.e, 63);
                const float cand = el * sig;
                const bool renorm = !(cand >= kSigMin);
                const float rn = renorm ? cand : 1.f;
                const float sig_new = renorm ? 1.f : cand;
                float *gH = reinterpret_cast<float *>(buf + L::oGate);
                if constexpr (P::kBF16) {
                    gH[lane] = gt.h * 1.4426950408889634f;   // log2(e)
                } else {
                    gH[lane] = gt.h;                         // H = h + lo, natural units
                    gH[7 * CH + lane] = gt.lo;
                }
                gH[CH + lane] = gt.e * sig;
                gH[2 * CH + lane] = gt.b;
                gH[3 * CH + lane] = gt.l / sig_new;
                gH[4 * CH + lane] = a.scale * (gt.e * sig);
                reinterpret_cast<int *>(gH + 5 * CH)[lane] = gt.rho;
                if (lane == 0) {
                    gH[6 * CH] = rn;
                    gH[6 * CH + 1] = sig_new;
                }
                sig = sig_new;
            }
            fetch((cc + 1) * CH);
            __builtin_amdgcn_s_setprio(0);
            prep_sync(pctr, target, lane, pfail);

            switch (pw) {
            case 0: prep_tiles<0, DK, P, WITH_O, L>(buf, smem, bo, lane, a.scale); break;
            case 1: prep_tiles<1, DK, P, WITH_O, L>(buf, smem, bo, lane, a.scale); break;
            case 2: prep_tiles<2, DK, P, WITH_O, L>(buf, smem, bo, lane, a.scale); break;
            case 3: prep_tiles<3, DK, P, WITH_O, L>(buf, smem, bo, lane, a.scale); break;
            case 4: prep_tiles<4, DK, P, WITH_O, L, HELP ? 1 : 2>(buf, smem, bo, lane, a.scale); break;
            case 5: prep_tiles<5, DK, P, WITH_O, L, HELP ? 1 : 2>(buf, smem, bo, lane, a.scale); break;
            case 6: prep_tiles<6, DK, P, WITH_O, L, HELP ? 1 : 2>(buf, smem, bo, lane, a.scale); break;
            default: break;
            }
            if (pw == GW) gt = gate_scan<!P::kBF16>(__uint_as_float(gpf), __uint_as_float(bpf), lane);
        };

        if (nch > 0) {
            fetch(0);
            if (pw == GW) gt = gate_scan<!P::kBF16>(__uint_as_float(gpf), __uint_as_float(bpf), lane);
            prep(0);
        }
        sync_lds();                                  // chunk 0 prepared
        for (int64_t c = 0; c < nch; ++c) {
            if (c + 1 < nch) prep(c + 1);
            sync_lds();
        }
        if (*pfail && lane == 0 && pw == 0) atomicOr(a.status, kStatusBitWait);
    }
}

// Workgroups of this kernel instance that can be resident at once on the current
// device (compute units x blocks per unit), queried once per device.
template <int DK, int DV, int W, class P, bool WITH_O>
int64_t resident_slots()
{
    static std::atomic<int64_t> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int64_t v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per, reinterpret_cast<const void *>(&gdn_chunk_ws_kernel<DK, DV, W, P, WITH_O, false>),
            64 * (W / 16 + NPW), 0) != hipSuccess)
        return 0;
    v = (int64_t)cus * (per > 0 ? per : 1);
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

template <int DK, int DV, int W, class P, bool WITH_O, bool MP = false>
hipError_t launch_t(const ChunkArgs &a0, hipStream_t stream)
{
    const int64_t units = (int64_t)a0.n_seqs * a0.h_v * (MP ? 2 : 1) * (DV / W);
    if (units <= 0) return hipSuccess;
    // split the units of a partial last round into column slices (2^split each, at least
    // 16 columns) while they still fit in one round
    ChunkArgs a = a0;
    a.n_full = units;
    a.split = 0;
    const int64_t slots = resident_slots<DK, DV, W, P, WITH_O>();
    if (slots > 0) {
        const int64_t rem = units % slots;
        int sp = 0;
        while (rem > 0 && (16 << (sp + 1)) <= W && rem * (int64_t(2) << sp) <= slots) ++sp;
        if (sp > 0) {
            a.n_full = units - rem;
            a.split = sp;
        }
    }
    const int64_t nblk = a.n_full + ((units - a.n_full) << a.split);
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // when every unit is sliced and at least three state waves of a slice have no
    // columns, the slices run the variant whose idle state waves help with the Gram
    // tiles (a launch with whole units too keeps one dispatch: the slices' help did not
    // change its time)
    const bool help = a.n_full == 0 && a.split > 0 && W / 16 - ((W >> a.split) / 16) >= 3;
    if (!help) {
        hipLaunchKernelGGL((gdn_chunk_ws_kernel<DK, DV, W, P, WITH_O, false, MP>), dim3((unsigned)nblk),
                           dim3(64 * (W / 16 + NPW)), 0, stream, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gdn_chunk_ws_kernel<DK, DV, W, P, WITH_O, true, MP>), dim3((unsigned)nblk),
                       dim3(64 * (W / 16 + NPW)), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_ws(const ChunkArgs &a, int bf16, int d_k, int d_v, bool with_o, hipStream_t s)
{
#define GDN_DISPATCH(DK, DV, W, POL)                                                   \
    return with_o ? launch_t<DK, DV, W, POL, true>(a, s) : launch_t<DK, DV, W, POL, false>(a, s)
    if (a.mpart) {   // state and transition-map units of square states, no outputs
        if (with_o || d_k != d_v) return hipErrorNotSupported;
        if (bf16) {
            if (d_k == 128) return launch_t<128, 128, 128, PolBF16, false, true>(a, s);
            if (d_k == 64) return launch_t<64, 64, 64, PolBF16, false, true>(a, s);
        } else {
            if (d_k == 128) return launch_t<128, 128, 64, PolF32, false, true>(a, s);
            if (d_k == 64) return launch_t<64, 64, 64, PolF32, false, true>(a, s);
        }
        return hipErrorNotSupported;
    }
    if (bf16) {
        if (d_k == 128 && d_v == 128) GDN_DISPATCH(128, 128, 128, PolBF16);
        if (d_k == 64 && d_v == 64) GDN_DISPATCH(64, 64, 64, PolBF16);
        if (d_k == 128 && d_v == 64) GDN_DISPATCH(128, 64, 64, PolBF16);
        if (d_k == 64 && d_v == 128) GDN_DISPATCH(64, 128, 128, PolBF16);
    } else {
        if (d_k == 64 && d_v == 64) GDN_DISPATCH(64, 64, 64, PolF32);
        if (d_k == 64 && d_v == 128) GDN_DISPATCH(64, 128, 64, PolF32);
        if (d_k == 128 && d_v == 64) GDN_DISPATCH(128, 64, 64, PolF32);
        if (d_k == 128 && d_v == 128) GDN_DISPATCH(128, 128, 64, PolF32);
    }
#undef GDN_DISPATCH
    return hipErrorNotSupported;
}

}  // namespace gdn
