// Chunked gated delta rule (replay and prefill) for gfx950 / CDNA4.
//
// The recurrence (Gated DeltaNet, as replayed by Tail-Replay over the last r tokens
// of a matched prefix from a zero state; gist.science technical summary,
// "Mecanismos Principais"):
//     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,   o_t = scale S_t^T q_t
// is evaluated in chunks of C = 64 tokens.  For one chunk with incoming state S:
//     H_i  cumulative log-gate since the last a = 0 token,  e_i = exp(H_i) (0 after a reset)
//     G_ij = exp(H_i - H_j) if no reset in (j, i], else 0             (j <= i)
//     A    = strict_lower(diag(b) (K K^T o G)),   T = (I + A)^{-1}   (UT transform)
//     X    = K S,  Y = diag(b) (V - diag(e) X),  U = T Y               (pseudo-values)
//     O    = scale (diag(e) Q S + lower(Q K^T o G) U)
//     S   <- e_last S + K^T diag(G_last,.) U
// which equals the token recurrence exactly in exact arithmetic.
//
// Work decomposition: one workgroup (4 waves) per (sequence, v-head, d_v block).
// The workgroup walks the chunks of its window in order; S (d_k x W fp32) never
// leaves the MFMA accumulators.  Each wave owns W/4 columns of S, which evolve
// independently because (I - b k k^T) acts on the d_k side only, so the state pass
// needs no cross-wave exchange.  The chunk-local operands (K, K^T, Q, T, P) are
// built once per chunk in LDS and shared by the four waves.
//
// Precision (bf16 inputs, fp32 state): q/k/v enter MFMA exactly; the gates, b, the
// unit diagonal of T and the diagonal of P are applied in fp32; S, U and P enter
// the products that feed o and S as hi+lo bf16 pairs; the UT inverse is computed in
// fp32 MFMA and rounded once.  fp32 inputs use fp32 MFMA throughout.
//
// Matrix-core layout used (16x16 MFMA): lane l supplies row l%16 of A and column
// l%16 of B; element j of lane group l/16 in A pairs with element j of the same
// lane group in B; the accumulator holds D[4*(l/16)+i][l%16] in element i.  A
// fragment whose contraction indices follow the accumulator rows lets a D tile be
// used directly as a B operand (S in K S, Y in T Y, U in P U and K^T U).
#include <type_traits>

#include "gdn_common.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int CH = 64;       // chunk length (tokens)
constexpr int LDF = CH + 4;  // row stride of the fp32 64x64 scratch matrices
constexpr int LDX = 16 + 4;  // row stride of a 16x16 fp32 scratch tile

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 h = (__bf16)f;                  // round to nearest even (v_cvt_pk_bf16_f32)
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// ---------------------------------------------------------------- policies
struct PolF32 {
    static constexpr bool kBF16 = false;
    static constexpr int KB = 16;    // contraction length of one fragment step
    static constexpr int PAD = 4;    // LDS row padding in elements (16 B)
    typedef float E;                 // element type of q/k/v and of LDS operands
    typedef f32x4 Frag;
};
struct PolBF16 {
    static constexpr bool kBF16 = true;
    static constexpr int KB = 32;
    static constexpr int PAD = 8;
    typedef uint16_t E;
    typedef bf16x8 Frag;
};

__device__ __forceinline__ f32x4 mma(f32x4 c, f32x4 a, f32x4 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}
__device__ __forceinline__ f32x4 mma(f32x4 c, bf16x8 a, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Fragment of a row-major LDS matrix M: lane l gives row r0 + l%16 and the
// contraction indices {4*(l/16) + i} (+16 for bf16) of k-block kb.
__device__ __forceinline__ f32x4 frag_rows(const float *M, int ld, int r0, int kb, int lane) {
    const float *p = M + (r0 + (lane & 15)) * ld + kb * 16 + 4 * (lane >> 4);
    return *reinterpret_cast<const f32x4 *>(p);
}
__device__ __forceinline__ bf16x8 frag_rows(const uint16_t *M, int ld, int r0, int kb, int lane) {
    const uint16_t *p = M + (r0 + (lane & 15)) * ld + kb * 32 + 4 * (lane >> 4);
    const u32x2 a = *reinterpret_cast<const u32x2 *>(p);
    const u32x2 b = *reinterpret_cast<const u32x2 *>(p + 16);
    const u32x4 u = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, u);
}
// fp32 fragment of M^T where M is row-major with the contraction index as its row:
// lane l gives column c0 + l%16, rows kb*16 + 4*(l/16) + i.
__device__ __forceinline__ f32x4 frag_cols(const float *M, int ld, int c0, int kb, int lane) {
    const int c = c0 + (lane & 15), k = kb * 16 + 4 * (lane >> 4);
    f32x4 f;
    f[0] = M[(k + 0) * ld + c];
    f[1] = M[(k + 1) * ld + c];
    f[2] = M[(k + 2) * ld + c];
    f[3] = M[(k + 3) * ld + c];
    return f;
}

// B operand from accumulator tiles covering one k-block (fp32: one tile).
__device__ __forceinline__ f32x4 bfrag(const f32x4 &t0, const f32x4 &) { return t0; }
__device__ __forceinline__ void bfrag_split(const f32x4 &t0, const f32x4 &, f32x4 &hi, f32x4 &lo) {
    hi = t0;
    lo = f32x4{0.f, 0.f, 0.f, 0.f};
}
// bf16: tiles t0 (block rows 0..15) and t1 (rows 16..31).
__device__ __forceinline__ bf16x8 bfrag_hi(const f32x4 &t0, const f32x4 &t1) {
    const u32x4 u = {pack2(t0[0], t0[1]), pack2(t0[2], t0[3]), pack2(t1[0], t1[1]),
                     pack2(t1[2], t1[3])};
    return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ void bfrag_split(const f32x4 &t0, const f32x4 &t1, bf16x8 &hi,
                                            bf16x8 &lo) {
    float h[8], r[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = bf2f(f2bf(t0[i]));
        h[4 + i] = bf2f(f2bf(t1[i]));
        r[i] = t0[i] - h[i];
        r[4 + i] = t1[i] - h[4 + i];
    }
    const u32x4 uh = {pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
    const u32x4 ul = {pack2(r[0], r[1]), pack2(r[2], r[3]), pack2(r[4], r[5]), pack2(r[6], r[7])};
    hi = __builtin_bit_cast(bf16x8, uh);
    lo = __builtin_bit_cast(bf16x8, ul);
}

template <class P>
__device__ __forceinline__ typename P::Frag bfrag_any(const f32x4 &t0, const f32x4 &t1) {
    if constexpr (P::kBF16) return bfrag_hi(t0, t1);
    else return t0;
}

__device__ __forceinline__ float ld_in(const float *p) { return *p; }
__device__ __forceinline__ float ld_in(const uint16_t *p) { return bf2f(*p); }
__device__ __forceinline__ void st_op(float *p, float x) { *p = x; }
__device__ __forceinline__ void st_op(uint16_t *p, float x) { *p = f2bf(x); }


__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(uint16_t x) { return bf2f(x); }


// A fragment read from a fp32 64-column LDS matrix (row stride LDF), converted to the
// operand type of the policy.
template <class P>
__device__ __forceinline__ typename P::Frag afrag_f32(const float *M, int r0, int kb, int lane) {
    const int row = r0 + (lane & 15);
    if constexpr (P::kBF16) {
        const int k0 = kb * 32 + 4 * (lane >> 4);
        const f32x4 x = *reinterpret_cast<const f32x4 *>(M + row * LDF + k0);
        const f32x4 y = *reinterpret_cast<const f32x4 *>(M + row * LDF + k0 + 16);
        const u32x4 u = {pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(y[0], y[1]), pack2(y[2], y[3])};
        return __builtin_bit_cast(bf16x8, u);
    } else {
        return *reinterpret_cast<const f32x4 *>(M + row * LDF + kb * 16 + 4 * (lane >> 4));
    }
}

// Row-contiguous store of a staged chunk of outputs (rows < len) for one v-head.
template <class E, int DV, int W, int NVO, int NTHR, int LDO>
__device__ __forceinline__ void store_o(const ChunkArgs &a, const E *Os, int64_t obase, int len,
                                        int h, int cb, int tid) {
    constexpr int VEC = 16 / (int)sizeof(E);
    E *og = reinterpret_cast<E *>(a.o_out);
#pragma unroll
    for (int j = 0; j < (CH * NVO) / NTHR; ++j) {
        const int e = tid + j * NTHR;
        const int rr = e / NVO, vc = e % NVO;
        if (rr < len)
            *reinterpret_cast<u32x4 *>(og + ((obase + rr) * a.h_v + h) * DV + cb * W + VEC * vc) =
                *reinterpret_cast<const u32x4 *>(Os + rr * LDO + VEC * vc);
    }
}

// V held in registers between its load and Y, one element per register.
template <class P> struct VHold {
    typedef typename std::conditional<P::kBF16, uint32_t, float>::type T;
    static constexpr int N = 4;
};

// Rows r0..r0+3 of column col of v-head h; rows past the chunk end read the last valid
// row (finite data that padded rows never use: their beta is 0).  No branches, so the
// loads stay in flight until Y consumes them.
template <class P>
__device__ __forceinline__ void load_v_rows(typename VHold<P>::T *out, const typename P::E *vg,
                                            int64_t t0, int r0, int len, int h_v, int h, int dv, int col) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = min(r0 + i, len - 1);
        if constexpr (P::kBF16) out[i] = (uint32_t)vg[((t0 + row) * h_v + h) * dv + col];
        else out[i] = vg[((t0 + row) * h_v + h) * dv + col];
    }
}
template <class P>
__device__ __forceinline__ float v_at(const typename VHold<P>::T *v, int i) {
    if constexpr (P::kBF16) return __uint_as_float(v[i] << 16);
    else return v[i];
}


// One lower-triangular 16x16 tile (ti, tj) of a chunk Gram product and its use:
//   K K^T tile -> -A = -b_r G_rc (K K^T)_rc  (fp32, c < r)
//   Q K^T tile ->  P = G_rc (Q K^T)_rc (c < r) and its diagonal (Q K^T)_rr
// with G_rc = exp(H_r - H_c) when no alpha = 0 token lies in (c, r].
template <class P, int KBK, int LDK, int LDP>
__device__ __forceinline__ void gram_tile(bool isP, int ti, int tj, const typename P::E *Ks,
                                          const typename P::E *Qs, float *nA, typename P::E *Ph,
                                          typename P::E *Pl, const float *gH, const float *gB,
                                          const int *gR, float *gPd, int lane) {
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 gr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KBK; ++kb)
        gr = mma(gr, frag_rows(isP ? Qs : Ks, LDK, 16 * ti, kb, lane), frag_rows(Ks, LDK, 16 * tj, kb, lane));
    const int c = 16 * tj + lr;
    const float hc = gH[c];
    const f32x4 hr = *reinterpret_cast<const f32x4 *>(gH + 16 * ti + 4 * lg);
    const f32x4 br = *reinterpret_cast<const f32x4 *>(gB + 16 * ti + 4 * lg);
    const int4 rr4 = *reinterpret_cast<const int4 *>(gR + 16 * ti + 4 * lg);
    const int rrs[4] = {rr4.x, rr4.y, rr4.z, rr4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = 16 * ti + 4 * lg + i;
        const float gam = (c < rr && rrs[i] <= c) ? __expf(hr[i] - hc) : 0.f;
        if (!isP) {
            nA[rr * LDF + c] = -br[i] * gam * gr[i];
        } else {
            const float pv = gam * gr[i];
            if constexpr (P::kBF16) {
                const uint16_t hb = f2bf(pv);
                Ph[rr * LDP + c] = hb;
                Pl[rr * LDP + c] = f2bf(pv - bf2f(hb));
            } else {
                Ph[rr * LDP + c] = pv;
            }
            if (c == rr) gPd[rr] = gr[i];
        }
    }
}

// Workgroup barrier that orders LDS only: global loads stay in flight across it
// (a full __syncthreads also waits for every outstanding global load).
__device__ __forceinline__ void sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Lower-triangular 16x16 tile list of a 64x64 product (ti >= tj).
__device__ __forceinline__ void tri_tile(int idx, int &ti, int &tj) {
    // 0:(0,0) 1:(1,0) 2:(1,1) 3:(2,0) 4:(2,1) 5:(2,2) 6:(3,0) 7:(3,1) 8:(3,2) 9:(3,3)
    ti = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
    tj = idx - (ti * (ti + 1)) / 2;
}

// ---------------------------------------------------------------- LDS plan
// One workgroup per CU; every region has a single role within a chunk:
//   G  gate arrays (first, so their offsets fit the DS immediate)
//   K  K chunk, row-major         Q  Q chunk, row-major       Kt  K^T (bf16 only)
//   A  -A (fp32)                  T  block-diagonal inverses T_bb - I (fp32)
//   P  P = strict_lower(Q K^T o G) (bf16 hi + lo, or fp32)    O  output staging
template <int DK, int DV, int W, class P>
struct Lds {
    typedef typename P::E E;
    static constexpr int LDK = DK + P::PAD;          // K, Q rows
    static constexpr int LDO = W + P::PAD;           // O staging rows
    static constexpr int LDKT = CH + 4;              // K^T rows (bf16)
    static constexpr int LDP = CH + P::PAD;          // P rows
    static constexpr int oG = 0;
    static constexpr int oK = 6 * CH * 4 + 64;
    static constexpr int oQ = oK + CH * LDK * (int)sizeof(E);
    static constexpr int oKt = oQ + CH * LDK * (int)sizeof(E);
    static constexpr int oA = oKt + (P::kBF16 ? DK * LDKT * 2 : 0);
    static constexpr int oT = oA + CH * LDF * 4;
    static constexpr int oP = oT + CH * LDF * 4;
    static constexpr int oO = oP + (P::kBF16 ? 2 : 1) * CH * LDP * (int)sizeof(E);
    static constexpr int bytes = oO + CH * LDO * (int)sizeof(E);
};

// ---------------------------------------------------------------- kernel
template <int DK, int DV, int W, class P, bool WITH_O>
__global__ void __launch_bounds__(64 * (W / 16)) gdn_chunk_kernel(ChunkArgs a)
{
    constexpr int NWAVE = W / 16;          // one 16-column tile of S per wave
    constexpr int NTHR = 64 * NWAVE;
    typedef typename P::E E;
    typedef typename P::Frag Frag;
    typedef Lds<DK, DV, W, P> L;
    constexpr int RT = DK / 16;            // row tiles of S
    constexpr int KBK = DK / P::KB;        // k-blocks over d_k
    constexpr int KBT = CH / P::KB;        // k-blocks over the chunk's tokens
    constexpr int NCB = DV / W;            // column blocks per head
    static_assert(L::bytes <= 160 * 1024, "LDS plan");

    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    E *Ks = reinterpret_cast<E *>(smem + L::oK);
    E *Qs = reinterpret_cast<E *>(smem + L::oQ);
    uint16_t *Kt = reinterpret_cast<uint16_t *>(smem + L::oKt);
    float *nA = reinterpret_cast<float *>(smem + L::oA);
    float *Tb = reinterpret_cast<float *>(smem + L::oT);
    E *Ph = reinterpret_cast<E *>(smem + L::oP);
    E *Pl = Ph + CH * L::LDP;
    E *Os = reinterpret_cast<E *>(smem + L::oO);
    float *gH = reinterpret_cast<float *>(smem + L::oG);   // cumulative log-gate since last reset
    float *gE = gH + CH;       // e_i
    float *gB = gE + CH;       // beta_i
    float *gL = gB + CH;       // G_last,i
    float *gPd = gL + CH;      // (Q K^T)_ii
    int *gR = reinterpret_cast<int *>(gPd + CH);   // last reset index at or before i
    int64_t *gMisc = reinterpret_cast<int64_t *>(gR + CH);

    const int tid0 = threadIdx.x, wave = tid0 >> 6;
    int tid = tid0, lane = tid0 & 63, lr = lane & 15, lg = lane >> 4;

    // ---- block -> (sequence, v-head, column block); XCD-aware: consecutive logical
    // blocks (the v-heads of one q/k head, the heads of one sequence) share an XCD's L2.
    const int64_t nblk = (int64_t)gridDim.x;
    int64_t bid = blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int cb = (int)(bid % NCB);
    const int h = (int)((bid / NCB) % a.h_v);
    const int n = (int)(bid / ((int64_t)NCB * a.h_v));
    const int hk = (int)(((int64_t)h * a.h_qk) / a.h_v);
    const bool replay = a.r != nullptr;

    // ---- window selection (validates the device-resident cu_seqlens / r)
    if (bid == 0) {
        int bad = 0;
        for (int m = tid; m < a.n_seqs; m += NTHR) {
            const int64_t b0 = a.cu[m], b1 = a.cu[m + 1];
            if (b0 < 0 || b1 < b0 || b1 > a.total_tokens) bad = 1;
            if (replay && (a.r[m] < 0 || a.r[m] > b1 - b0)) bad = 1;
        }
        if (replay && wave == 0) {   // the packed outputs must fit o_out
            int64_t tot = 0;
            for (int m = lane; m < a.n_seqs; m += 64) tot += a.r[m];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
            if (tot > a.total_out) bad = 1;
        }
        bad = __syncthreads_or(bad);
        if (tid == 0) *a.status = bad ? kStatusBadInput : kStatusOk;
    }
    const int64_t beg = a.cu[n], end = a.cu[n + 1];
    if (beg < 0 || end < beg || end > a.total_tokens) return;
    const int64_t rn = replay ? (int64_t)a.r[n] : end - beg;
    if (rn < 0 || rn > end - beg) return;
    const int64_t wbeg = end - rn;              // first token of the window
    if (wave == 0) {
        int64_t row0 = beg;
        if (replay) {
            int64_t s = 0;
            for (int m = lane; m < n; m += 64) s += a.r[m];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
            row0 = s;
        }
        if (lane == 0) gMisc[0] = row0;
    }
    // T_bb regions outside the diagonal blocks are read (and multiplied by zeros):
    // keep them finite
    for (int e = tid; e < CH * LDF; e += NTHR) Tb[e] = 0.f;
    __syncthreads();
    const int64_t orow0 = gMisc[0];
    if (orow0 < 0 || orow0 + rn > (replay ? a.total_out : a.total_tokens)) return;
    if (a.cu_out && h == 0 && cb == 0 && tid == 0) {
        a.cu_out[n] = (int32_t)orow0;
        if (n == a.n_seqs - 1) a.cu_out[n + 1] = (int32_t)(orow0 + rn);
    }

    const int col0 = cb * W + wave * 16;       // first d_v column of this wave
    const int64_t sbase = ((int64_t)n * a.h_v + h) * DK * DV;

    // ---- state: S[rt] holds rows 16rt.. of columns col0..col0+15
    f32x4 S[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (!replay && a.S0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[rt][i] = a.S0[sbase + (int64_t)(16 * rt + 4 * lg + i) * DV + col0 + lr];
        } else {
            S[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    const E *qg = reinterpret_cast<const E *>(a.q);
    const E *kg = reinterpret_cast<const E *>(a.k);
    const E *vg = reinterpret_cast<const E *>(a.v);
    constexpr int VEC = 16 / (int)sizeof(E);   // elements per 16-byte vector
    constexpr int NVK = DK / VEC;              // vectors per K/Q row
    constexpr int NVO = W / VEC;               // vectors per O row (this column block)
    static_assert(NVK <= 64 && (64 % NVK) == 0 && (CH * NVO) % NTHR == 0, "vector maps");

    constexpr int RPP = NTHR / NVK;            // K/Q rows per pass of the workgroup
    constexpr int NPF = CH / RPP;              // passes per chunk
    u32x4 kpf[NPF], qpf[NPF];
    float gpf = 0.f, bpf = 0.f;
    bool gok = false;
    typename VHold<P>::T vnext[4][VHold<P>::N];
    auto fetch = [&](int64_t cc) {
        const int ln = (int)((rn - cc) < CH ? (rn - cc) : CH);
        const int64_t tb = wbeg + cc;
        // rows past the chunk end load the last valid row: finite, and inert because
        // their g and beta are set to 0 (alpha = 1, no write)
#pragma unroll
        for (int p = 0; p < NPF; ++p) {
            const int row = min(p * RPP + tid / NVK, ln - 1);
            const int64_t off = ((tb + row) * a.h_qk + hk) * DK + (int64_t)(tid % NVK) * VEC;
            kpf[p] = *reinterpret_cast<const u32x4 *>(kg + off);
            if (WITH_O) qpf[p] = *reinterpret_cast<const u32x4 *>(qg + off);
        }
        {
            const int64_t off = (tb + min(lane, ln - 1)) * a.h_v + h;
            gpf = a.g[off];
            bpf = a.beta[off];
            gok = lane < ln;
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
            load_v_rows<P>(vnext[tt], vg, tb, 16 * tt + 4 * lg, ln, a.h_v, h, DV, col0 + lr);
    };
    if (rn > 0) fetch(0);

    int64_t opend = -1;        // first output row of the chunk staged in Os, if any
    int olen = 0;
    for (int64_t c0 = 0; c0 < rn; c0 += CH) {
        const int len = (int)((rn - c0) < CH ? (rn - c0) : CH);
        const int64_t t0 = wbeg + c0;
        // lane-derived indices are recomputed each chunk instead of being held in
        // registers across the whole loop
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
        sync_lds();

        // ================= P0: store the previous chunk's staged outputs; this chunk's
        // K, Q into LDS (prefetched during the previous chunk); gate scan.
        // Rows >= len repeat the last token's q/k/v but get g = 0 and beta = 0: a token
        // with alpha = 1 and no write leaves S unchanged, and its pseudo-value is 0.
        if constexpr (WITH_O) {
            if (opend >= 0) store_o<E, DV, W, NVO, NTHR, L::LDO>(a, Os, opend, olen, h, cb, tid);
        }
#pragma unroll
        for (int p = 0; p < NPF; ++p) {
            const int row = p * RPP + tid / NVK;
            *reinterpret_cast<u32x4 *>(Ks + row * L::LDK + (tid % NVK) * VEC) = kpf[p];
            if (WITH_O) *reinterpret_cast<u32x4 *>(Qs + row * L::LDK + (tid % NVK) * VEC) = qpf[p];
        }
        if (wave == 0) {
            const float gv = gok ? gpf : 0.f, bv = gok ? bpf : 0.f;
            // reset-aware inclusive scan: H = sum of g since the last alpha = 0 token
            const bool reset = gv == -__builtin_inff();
            float hv = reset ? 0.f : gv;
            int seg = reset ? 1 : 0;
            int rho = reset ? lane : -1;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float ho = __shfl_up(hv, off);
                const int so = __shfl_up(seg, off);
                const int ro = __shfl_up(rho, off);
                if (lane >= off) {
                    if (!seg) hv += ho;
                    seg |= so;
                    rho = ro > rho ? ro : rho;
                }
            }
            const float hl = __shfl(hv, 63);
            const int rl = __shfl(rho, 63);
            gH[lane] = hv;
            gE[lane] = rho < 0 ? __expf(hv) : 0.f;
            gB[lane] = bv;
            gR[lane] = rho;
            gL[lane] = rl <= lane ? __expf(hl - hv) : 0.f;
        }
        sync_lds();

        // ================= P1: X = K S and Q S (S as hi, hi + lo); the K K^T Gram tiles
        // forming -A = -strict_lower(diag(b) (K K^T o G)).
        f32x4 X[4], QS[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            X[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            QS[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < KBK; ++kb) {
            Frag sh, sl;
            if constexpr (P::kBF16) bfrag_split(S[2 * kb], S[2 * kb + 1], sh, sl);
            else sh = S[kb];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                X[tt] = mma(X[tt], frag_rows(Ks, L::LDK, 16 * tt, kb, lane), sh);
                if constexpr (WITH_O) {
                    const Frag qf = frag_rows(Qs, L::LDK, 16 * tt, kb, lane);
                    QS[tt] = mma(QS[tt], qf, sh);
                    if constexpr (P::kBF16) QS[tt] = mma(QS[tt], qf, sl);
                }
            }
        }
        {
            // the 10 K K^T tiles over the waves (two per wave when there are 4 waves)
            static_assert(NWAVE == 4 || NWAVE == 8, "tile schedule");
            int ti, tj;
            tri_tile(wave, ti, tj);
            gram_tile<P, KBK, L::LDK, L::LDP>(false, ti, tj, Ks, Qs, nA, Ph, Pl, gH, gB, gR, gPd, lane);
            if (wave + NWAVE < 10) {
                tri_tile(wave + NWAVE, ti, tj);
                gram_tile<P, KBK, L::LDK, L::LDP>(false, ti, tj, Ks, Qs, nA, Ph, Pl, gH, gB, gR, gPd, lane);
            }
            if (NWAVE == 4 && wave < 2) {
                tri_tile(wave + 8, ti, tj);
                gram_tile<P, KBK, L::LDK, L::LDP>(false, ti, tj, Ks, Qs, nA, Ph, Pl, gH, gB, gR, gPd, lane);
            }
        }
        sync_lds();

        // ================= P2: diagonal-block inverses T_bb = (I + A_bb)^{-1} by forward
        // substitution (first half of the waves, one column per lane), stored as T_bb - I;
        // P = strict_lower(Q K^T o G) and K^T (second half); Y = b (V - e X) (every wave);
        // then the next chunk's inputs are fetched.
        if (wave < 4 && lane < 16) {
            const int b0 = 16 * wave;
            const int c = lane;
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) s = fmaf(nA[(b0 + i) * LDF + b0 + j], t[j], s);
                t[i] = i < c ? 0.f : (i == c ? 1.f : s);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) Tb[(b0 + i) * LDF + b0 + c] = i == c ? 0.f : t[i];
        }
        if (wave >= NWAVE / 2) {
            // the other half of the waves: the 10 Q K^T tiles (P) and K^T, while the
            // first half inverts the diagonal blocks
            const int w2 = wave - NWAVE / 2;            // 0..NWAVE/2-1
            if constexpr (WITH_O) {
#pragma unroll
                for (int j = 0; j < (10 + NWAVE / 2 - 1) / (NWAVE / 2); ++j) {
                    const int idx = w2 + (NWAVE / 2) * j;
                    if (idx < 10) {
                        int ti, tj;
                        tri_tile(idx, ti, tj);
                        gram_tile<P, KBK, L::LDK, L::LDP>(true, ti, tj, Ks, Qs, nA, Ph, Pl, gH, gB, gR, gPd, lane);
                    }
                }
                if (P::kBF16 && w2 < 2) {
                    // zero the upper tiles (0,1) and (2,3) that 32-wide k-blocks of P read
                    const int ti = 2 * w2, tj = ti + 1;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = 16 * ti + 4 * lg + i, c = 16 * tj + lr;
                        Ph[rr * L::LDP + c] = 0;
                        Pl[rr * L::LDP + c] = 0;
                    }
                }
            }
            if constexpr (P::kBF16) {
                // K^T[dk][t] as packed token pairs: thread -> (token pair, 8-column block)
                constexpr int NCB8 = DK / 8;
                static_assert((32 * NCB8) % (NTHR / 2) == 0 || (NTHR / 2) % (32 * NCB8) == 0, "K^T map");
#pragma unroll
                for (int j = 0; j < (32 * NCB8 + NTHR / 2 - 1) / (NTHR / 2); ++j) {
                    const int u = (tid - NTHR / 2) + j * (NTHR / 2);
                    if (u < 32 * NCB8) {
                        const int pr = u & 31, c8 = u >> 5;
                        const u32x4 x0 = *reinterpret_cast<const u32x4 *>(Ks + (2 * pr) * L::LDK + 8 * c8);
                        const u32x4 x1 = *reinterpret_cast<const u32x4 *>(Ks + (2 * pr + 1) * L::LDK + 8 * c8);
                        const uint32_t xs0[4] = {x0.x, x0.y, x0.z, x0.w}, xs1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t lo = (xs0[e] & 0xffffu) | (xs1[e] << 16);
                            const uint32_t hi = (xs0[e] >> 16) | (xs1[e] & 0xffff0000u);
                            *reinterpret_cast<uint32_t *>(Kt + (8 * c8 + 2 * e) * L::LDKT + 2 * pr) = lo;
                            *reinterpret_cast<uint32_t *>(Kt + (8 * c8 + 2 * e + 1) * L::LDKT + 2 * pr) = hi;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const f32x4 br = *reinterpret_cast<const f32x4 *>(gB + 16 * tt + 4 * lg);
            const f32x4 er = *reinterpret_cast<const f32x4 *>(gE + 16 * tt + 4 * lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) X[tt][i] = br[i] * (v_at<P>(vnext[tt], i) - er[i] * X[tt][i]);
        }
        // every input of this chunk is consumed: the next chunk's land while the rest of
        // this chunk is processed
        if (c0 + CH < rn) fetch(c0 + CH);
        sync_lds();

        // ================= P3: (I + A) U = Y by 16-row block forward substitution
        //   U_b = Z_b + (T_bb - I) Z_b,   Z_b = Y_b - sum_{j<b} A_bj U_j
        // (unit diagonal exact in fp32); then O and the state update.
        f32x4 U[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f32x4 z = X[b];
            if constexpr (P::kBF16) {
                if (b >= 1) {
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    z = mma(z, afrag_f32<P>(nA, 16 * b, 0, lane), bfrag_hi(U[0], b >= 2 ? U[1] : zero));
                    if (b == 3) z = mma(z, afrag_f32<P>(nA, 16 * b, 1, lane), bfrag_hi(U[2], zero));
                }
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const Frag zf = (b & 1) ? bfrag_hi(zero, z) : bfrag_hi(z, zero);
                U[b] = mma(z, afrag_f32<P>(Tb, 16 * b, b >> 1, lane), zf);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (j < b) z = mma(z, afrag_f32<P>(nA, 16 * b, j, lane), U[j]);
                U[b] = mma(z, afrag_f32<P>(Tb, 16 * b, b, lane), z);
            }
        }
        // O = e (Q S) + Pd U + P_off U   (QS registers become O)
        if constexpr (WITH_O) {
            Frag uh[KBT], ul[KBT];
#pragma unroll
            for (int kb = 0; kb < KBT; ++kb) {
                if constexpr (P::kBF16) bfrag_split(U[2 * kb], U[2 * kb + 1], uh[kb], ul[kb]);
                else uh[kb] = U[kb];
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const f32x4 er = *reinterpret_cast<const f32x4 *>(gE + 16 * tt + 4 * lg);
                const f32x4 pd = *reinterpret_cast<const f32x4 *>(gPd + 16 * tt + 4 * lg);
#pragma unroll
                for (int i = 0; i < 4; ++i) QS[tt][i] = er[i] * QS[tt][i] + pd[i] * U[tt][i];
#pragma unroll
                for (int kb = 0; kb < KBT; ++kb) {
                    if (kb * P::KB < 16 * tt + 16) {
                        const Frag ph = frag_rows(Ph, L::LDP, 16 * tt, kb, lane);
                        QS[tt] = mma(QS[tt], ph, uh[kb]);
                        if constexpr (P::kBF16) {
                            QS[tt] = mma(QS[tt], ph, ul[kb]);
                            QS[tt] = mma(QS[tt], frag_rows(Pl, L::LDP, 16 * tt, kb, lane), uh[kb]);
                        }
                    }
                }
            }
            const int64_t obase = replay ? orow0 + c0 : t0;
            if (a.o_out) {
                if (a.o_f32) {
                    float *og = reinterpret_cast<float *>(a.o_out);
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int rr = 16 * tt + 4 * lg + i;
                            if (rr < len) og[((obase + rr) * a.h_v + h) * DV + col0 + lr] = a.scale * QS[tt][i];
                        }
                } else {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            st_op(Os + (16 * tt + 4 * lg + i) * L::LDO + wave * 16 + lr, a.scale * QS[tt][i]);
                    opend = obase;
                    olen = len;
                }
            }
        }
        // S <- e_last S + K^T diag(G_last) U
        {
            const float gam_c = gE[CH - 1];
            Frag dh[KBT], dl[KBT];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const f32x4 l4 = *reinterpret_cast<const f32x4 *>(gL + 16 * tt + 4 * lg);
#pragma unroll
                for (int i = 0; i < 4; ++i) U[tt][i] *= l4[i];
            }
#pragma unroll
            for (int kb = 0; kb < KBT; ++kb) {
                if constexpr (P::kBF16) bfrag_split(U[2 * kb], U[2 * kb + 1], dh[kb], dl[kb]);
                else dh[kb] = U[kb];
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f32x4 s = S[rt] * gam_c;
#pragma unroll
                for (int kb = 0; kb < KBT; ++kb) {
                    if constexpr (P::kBF16) {
                        const Frag kf = frag_rows(Kt, L::LDKT, 16 * rt, kb, lane);
                        s = mma(s, kf, dh[kb]);
                        s = mma(s, kf, dl[kb]);
                    } else {
                        s = mma(s, frag_cols(reinterpret_cast<const float *>(Ks), L::LDK, 16 * rt, kb, lane), dh[kb]);
                    }
                }
                S[rt] = s;
            }
        }
    }
    if constexpr (WITH_O) {
        if (opend >= 0) {
            sync_lds();
            store_o<E, DV, W, NVO, NTHR, L::LDO>(a, Os, opend, olen, h, cb, tid);
        }
    }

    // ---- state write-back
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a.S_out[sbase + (int64_t)(16 * rt + 4 * lg + i) * DV + col0 + lr] = S[rt][i];
}

template <int DK, int DV, int W, class P, bool WITH_O>
hipError_t launch_t(const ChunkArgs &a, hipStream_t stream)
{
    const int64_t nblk = (int64_t)a.n_seqs * a.h_v * (DV / W);
    if (nblk <= 0) return hipSuccess;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gdn_chunk_kernel<DK, DV, W, P, WITH_O>), dim3((unsigned)nblk), dim3(64 * (W / 16)), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk(const ChunkArgs &a, int bf16, int d_k, int d_v, bool with_o, hipStream_t s)
{
#define GDN_DISPATCH(DK, DV, W, POL)                                                   \
    return with_o ? launch_t<DK, DV, W, POL, true>(a, s) : launch_t<DK, DV, W, POL, false>(a, s)
    if (bf16) {
        if (d_k == 128 && d_v == 128) GDN_DISPATCH(128, 128, 128, PolBF16);
        if (d_k == 64 && d_v == 64) GDN_DISPATCH(64, 64, 64, PolBF16);
        if (d_k == 128 && d_v == 64) GDN_DISPATCH(128, 64, 64, PolBF16);
        if (d_k == 64 && d_v == 128) GDN_DISPATCH(64, 128, 128, PolBF16);
    } else {
        if (d_k == 64 && d_v == 64) GDN_DISPATCH(64, 64, 64, PolF32);
        if (d_k == 64 && d_v == 128) GDN_DISPATCH(64, 128, 64, PolF32);
    }
#undef GDN_DISPATCH
    return hipErrorNotSupported;
}

}  // namespace gdn
