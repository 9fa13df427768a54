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
#include "gdn_common.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int CH = 64;       // chunk length (tokens)
constexpr int NWAVE = 4;
constexpr int NTHR = 64 * NWAVE;
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

// Lower-triangular 16x16 tile list of a 64x64 product (ti >= tj).
__device__ __forceinline__ void tri_tile(int idx, int &ti, int &tj) {
    // 0:(0,0) 1:(1,0) 2:(1,1) 3:(2,0) 4:(2,1) 5:(2,2) 6:(3,0) 7:(3,1) 8:(3,2) 9:(3,3)
    ti = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
    tj = idx - (ti * (ti + 1)) / 2;
}

// ---------------------------------------------------------------- LDS plan
template <int DK, int DV, int W, class P>
struct Lds {
    typedef typename P::E E;
    static constexpr int LDK = DK + P::PAD;    // K, Q rows
    static constexpr int LDT = CH + P::PAD;    // K^T rows, T_off, P rows
    static constexpr int LDV = W + P::PAD;     // V and O staging rows
    static constexpr int oK = 0;
    static constexpr int oQ = oK + CH * LDK * (int)sizeof(E);
    static constexpr int oKt = oQ + CH * LDK * (int)sizeof(E);
    static constexpr int nKt = P::kBF16 ? DK * LDT * (int)sizeof(E) : 0;
    static constexpr int oV = oKt + nKt;
    static constexpr int oT = oV + CH * LDV * (int)sizeof(E);
    static constexpr int oPh = oT + CH * LDT * (int)sizeof(E);
    static constexpr int oPl = oPh + CH * LDT * (int)sizeof(E);
    static constexpr int nPl = P::kBF16 ? CH * LDT * (int)sizeof(E) : 0;
    static constexpr int oAf = oPl + nPl;                        // A (fp32); O staging aliases it
    static constexpr int nAf = CH * LDF * 4;
    static constexpr int nOs = CH * (W + 4) * 4;                 // worst case fp32 staging
    static constexpr int oTf = oAf + (nAf > nOs ? nAf : nOs);
    static constexpr int oXs = oTf + CH * LDF * 4;
    static constexpr int oGate = oXs + 4 * 16 * LDX * 4;
    static constexpr int bytes = oGate + 8 * CH * 4 + 64;
};

// ---------------------------------------------------------------- kernel
template <int DK, int DV, int W, class P, bool WITH_O>
__global__ void __launch_bounds__(NTHR) gdn_chunk_kernel(ChunkArgs a)
{
    typedef typename P::E E;
    typedef typename P::Frag Frag;
    typedef Lds<DK, DV, W, P> L;
    constexpr int WC = W / NWAVE;          // columns per wave
    constexpr int CT = WC / 16;            // column tiles per wave
    constexpr int RT = DK / 16;            // row tiles of S
    constexpr int KBK = DK / P::KB;        // k-blocks over d_k
    constexpr int KBT = CH / P::KB;        // k-blocks over the chunk's tokens
    constexpr int NCB = DV / W;            // column blocks per head
    static_assert(CT >= 1 && WC % 16 == 0, "wave column slab must be a multiple of 16");

    __shared__ __attribute__((aligned(16))) char smem[L::bytes];
    E *Ks = reinterpret_cast<E *>(smem + L::oK);
    E *Qs = reinterpret_cast<E *>(smem + L::oQ);
    E *Kt = reinterpret_cast<E *>(smem + L::oKt);
    E *Vs = reinterpret_cast<E *>(smem + L::oV);
    E *Ts = reinterpret_cast<E *>(smem + L::oT);
    E *Ph = reinterpret_cast<E *>(smem + L::oPh);
    E *Pl = reinterpret_cast<E *>(smem + L::oPl);
    float *Af = reinterpret_cast<float *>(smem + L::oAf);
    E *Os = reinterpret_cast<E *>(smem + L::oAf);
    float *Osf = reinterpret_cast<float *>(smem + L::oAf);
    float *Tf = reinterpret_cast<float *>(smem + L::oTf);
    float *Xs = reinterpret_cast<float *>(smem + L::oXs);
    float *gG = reinterpret_cast<float *>(smem + L::oGate);   // raw g, then H
    float *gE = gG + CH;       // e_i
    float *gB = gE + CH;       // beta_i
    float *gL = gB + CH;       // G_last,i
    float *gPd = gL + CH;      // (Q K^T)_ii
    int *gR = reinterpret_cast<int *>(gPd + CH);   // last reset index at or before i
    int64_t *gMisc = reinterpret_cast<int64_t *>(gR + CH);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

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
    __syncthreads();
    const int64_t orow0 = gMisc[0];
    if (orow0 < 0 || orow0 + rn > (replay ? a.total_out : a.total_tokens)) return;
    if (a.cu_out && h == 0 && cb == 0 && tid == 0) {
        a.cu_out[n] = (int32_t)orow0;
        if (n == a.n_seqs - 1) a.cu_out[n + 1] = (int32_t)(orow0 + rn);
    }

    const int col0 = cb * W + wave * WC;       // first d_v column of this wave
    const int64_t sbase = ((int64_t)n * a.h_v + h) * DK * DV;

    // ---- state: S[rt][ct] holds rows 16rt.., columns col0 + 16ct..
    f32x4 S[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            if (!replay && a.S0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[rt][ct][i] = a.S0[sbase + (int64_t)(16 * rt + 4 * lg + i) * DV + col0 + 16 * ct + lr];
            } else {
                S[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }

    const E *qg = reinterpret_cast<const E *>(a.q);
    const E *kg = reinterpret_cast<const E *>(a.k);
    const E *vg = reinterpret_cast<const E *>(a.v);
    constexpr int VEC = 16 / (int)sizeof(E);   // elements per 16-byte vector
    constexpr int NVK = DK / VEC;              // vectors per K/Q row
    constexpr int NVV = W / VEC;               // vectors per V row (this column block)
    static_assert(NVK <= 64 && NVV <= 64 && (64 % NVK) == 0 && (64 % NVV) == 0, "vector map");

    for (int64_t c0 = 0; c0 < rn; c0 += CH) {
        const int len = (int)((rn - c0) < CH ? (rn - c0) : CH);
        const int64_t t0 = wbeg + c0;
        __syncthreads();

        // ================= load the chunk (rows >= len are zero; g = 0, b = 0 there)
        {
            constexpr int RPP = NTHR / NVK;            // rows per pass
            const int vc = tid % NVK, rsub = tid / NVK;
#pragma unroll
            for (int p = 0; p < CH / RPP; ++p) {
                const int row = p * RPP + rsub;
                u32x4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
                if (row < len) {
                    const int64_t off = ((t0 + row) * a.h_qk + hk) * DK + (int64_t)vc * VEC;
                    kv = *reinterpret_cast<const u32x4 *>(kg + off);
                    if (WITH_O) qv = *reinterpret_cast<const u32x4 *>(qg + off);
                }
                *reinterpret_cast<u32x4 *>(Ks + row * L::LDK + vc * VEC) = kv;
                if (WITH_O) *reinterpret_cast<u32x4 *>(Qs + row * L::LDK + vc * VEC) = qv;
                if constexpr (P::kBF16) {
                    // K^T: pack token pairs (2m, 2m+1) of one d_k index into a dword.
                    // Partner row is NVK lanes away (same wave since NVK <= 32).
                    const bool odd = (row & 1) != 0;
                    const uint32_t s0 = odd ? kv.x : kv.z, s1 = odd ? kv.y : kv.w;
                    const uint32_t r0 = (uint32_t)__shfl_xor((int)s0, NVK);
                    const uint32_t r1 = (uint32_t)__shfl_xor((int)s1, NVK);
                    const int rev = row & ~1;
                    uint32_t w0, w1, w2, w3;
                    int e0;
                    if (!odd) {   // my elements 0..3 (row 2m) + partner's 0..3 (row 2m+1)
                        w0 = (kv.x & 0xffffu) | (r0 << 16);
                        w1 = (kv.x >> 16) | (r0 & 0xffff0000u);
                        w2 = (kv.y & 0xffffu) | (r1 << 16);
                        w3 = (kv.y >> 16) | (r1 & 0xffff0000u);
                        e0 = 0;
                    } else {      // partner's elements 4..7 (row 2m) + my 4..7 (row 2m+1)
                        w0 = (r0 & 0xffffu) | (kv.z << 16);
                        w1 = (r0 >> 16) | (kv.z & 0xffff0000u);
                        w2 = (r1 & 0xffffu) | (kv.w << 16);
                        w3 = (r1 >> 16) | (kv.w & 0xffff0000u);
                        e0 = 4;
                    }
                    const int dk0 = vc * VEC + e0;
                    *reinterpret_cast<uint32_t *>(Kt + (dk0 + 0) * L::LDT + rev) = w0;
                    *reinterpret_cast<uint32_t *>(Kt + (dk0 + 1) * L::LDT + rev) = w1;
                    *reinterpret_cast<uint32_t *>(Kt + (dk0 + 2) * L::LDT + rev) = w2;
                    *reinterpret_cast<uint32_t *>(Kt + (dk0 + 3) * L::LDT + rev) = w3;
                }
            }
        }
        {
            constexpr int RPP = NTHR / NVV;
            const int vc = tid % NVV, rsub = tid / NVV;
#pragma unroll
            for (int p = 0; p < CH / RPP; ++p) {
                const int row = p * RPP + rsub;
                u32x4 vv = {0u, 0u, 0u, 0u};
                if (row < len) {
                    const int64_t off = ((t0 + row) * a.h_v + h) * DV + (int64_t)cb * W + vc * VEC;
                    vv = *reinterpret_cast<const u32x4 *>(vg + off);
                }
                *reinterpret_cast<u32x4 *>(Vs + row * L::LDV + vc * VEC) = vv;
            }
        }
        if (tid < CH) {
            float gv = 0.f, bv = 0.f;
            if (tid < len) {
                const int64_t off = (t0 + tid) * a.h_v + h;
                gv = a.g[off];
                bv = a.beta[off];
            }
            gG[tid] = gv;
            gB[tid] = bv;
        }
        __syncthreads();

        // ================= gates (wave 0): reset-aware segmented scan over the chunk
        if (wave == 0) {
            const float gv = gG[lane];
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
            gG[lane] = hv;
            gE[lane] = rho < 0 ? __expf(hv) : 0.f;
            gR[lane] = rho;
            gL[lane] = rl <= lane ? __expf(hl - hv) : 0.f;
        }

        // ================= Gram tiles: K K^T (tiles 0..9) and Q K^T (tiles 10..19)
        constexpr int NG = WITH_O ? 20 : 10;
        constexpr int GPW = (NG + NWAVE - 1) / NWAVE;
        f32x4 gram[GPW];
#pragma unroll
        for (int j = 0; j < GPW; ++j) {
            const int idx = wave + NWAVE * j;
            gram[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (idx < NG) {
                int ti, tj;
                tri_tile(idx % 10, ti, tj);
                const E *Am = idx < 10 ? Ks : Qs;
#pragma unroll
                for (int kb = 0; kb < KBK; ++kb)
                    gram[j] = mma(gram[j], frag_rows(Am, L::LDK, 16 * ti, kb, lane),
                                  frag_rows(Ks, L::LDK, 16 * tj, kb, lane));
            }
        }
        __syncthreads();

        // ================= A = strict_lower(diag(b) (K K^T o G)); P = lower(Q K^T o G)
#pragma unroll
        for (int j = 0; j < GPW; ++j) {
            const int idx = wave + NWAVE * j;
            if (idx < NG) {
                int ti, tj;
                tri_tile(idx % 10, ti, tj);
                const int c = 16 * tj + lr;
                const float hc = gG[c];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * ti + 4 * lg + i;
                    const float gam = (c <= rr && gR[rr] <= c) ? __expf(gG[rr] - hc) : 0.f;
                    const float x = gram[j][i];
                    if (idx < 10) {
                        Af[rr * LDF + c] = c < rr ? gB[rr] * gam * x : 0.f;
                    } else {
                        const float pv = c < rr ? gam * x : 0.f;
                        if constexpr (P::kBF16) {
                            const uint16_t hb = f2bf(pv);
                            Ph[rr * L::LDT + c] = hb;
                            Pl[rr * L::LDT + c] = f2bf(pv - bf2f(hb));
                        } else {
                            Ph[rr * L::LDT + c] = pv;
                        }
                        if (c == rr) gPd[rr] = x;
                    }
                }
            }
        }
        if (WITH_O && P::kBF16 && wave < 2) {
            // zero the upper tiles (0,1) and (2,3) read by 32-wide k-blocks of P
            const int ti = 2 * wave, tj = ti + 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * ti + 4 * lg + i, c = 16 * tj + lr;
                Ph[rr * L::LDT + c] = 0;
                Pl[rr * L::LDT + c] = 0;
            }
        }
        __syncthreads();

        // ================= T = (I + A)^{-1} in fp32 (blocked, 16x16 diagonal blocks)
        // level 0: wave b inverts diagonal block b by forward substitution (column = lane)
        if (lane < 16) {
            const int b0 = 16 * wave;
            const int c = lane;
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) s = fmaf(Af[(b0 + i) * LDF + b0 + j], t[j], s);
                t[i] = i < c ? 0.f : (i == c ? 1.f : -s);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) Tf[(b0 + i) * LDF + b0 + c] = t[i];
        }
        __syncthreads();
        // level 1: T_{b+1,b} = -T_{b+1,b+1} A_{b+1,b} T_{b,b} for b = 0 (wave 0), 2 (wave 1)
        if (wave < 2) {
            const int b = 2 * wave;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            x = mma(x, frag_rows(Af, LDF, 16 * (b + 1), b, lane), frag_cols(Tf, LDF, 16 * b, b, lane));
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            y = mma(y, frag_rows(Tf, LDF, 16 * (b + 1), b + 1, lane), x);
#pragma unroll
            for (int i = 0; i < 4; ++i) Tf[(16 * (b + 1) + 4 * lg + i) * LDF + 16 * b + lr] = -y[i];
        }
        __syncthreads();
        // level 2: lower-left 32x32 block = -T_lowerright A_21 T_upperleft
        const int la = wave >> 1, lb = wave & 1;
        {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 2; ++c)
                if (c >= lb)
                    x = mma(x, frag_rows(Af, LDF, 16 * (2 + la), c, lane),
                            frag_cols(Tf, LDF, 16 * lb, c, lane));
            float *X = Xs + (la * 2 + lb) * 16 * LDX;
#pragma unroll
            for (int i = 0; i < 4; ++i) X[(4 * lg + i) * LDX + lr] = x[i];
        }
        __syncthreads();
        {
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 0; d < 2; ++d)
                if (d <= la)
                    y = mma(y, frag_rows(Tf, LDF, 16 * (2 + la), 2 + d, lane),
                            frag_cols(Xs + (d * 2 + lb) * 16 * LDX, LDX, 0, 0, lane));
#pragma unroll
            for (int i = 0; i < 4; ++i) Tf[(16 * (2 + la) + 4 * lg + i) * LDF + 16 * lb + lr] = -y[i];
        }
        __syncthreads();
        // strictly lower part of T -> operand type (zeros elsewhere)
        for (int e = tid; e < CH * CH; e += NTHR) {
            const int rr = e >> 6, c = e & 63;
            st_op(Ts + rr * L::LDT + c, c < rr ? Tf[rr * LDF + c] : 0.f);
        }
        __syncthreads();

        // ================= state pass on this wave's columns
        const float gam_c = gE[CH - 1];
        // S fragments (hi and lo) over d_k
        Frag sh[KBK][CT], sl[KBK][CT];
#pragma unroll
        for (int kb = 0; kb < KBK; ++kb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                if constexpr (P::kBF16) bfrag_split(S[2 * kb][ct], S[2 * kb + 1][ct], sh[kb][ct], sl[kb][ct]);
                else sh[kb][ct] = S[kb][ct];
            }
        // X = K S ; Y = b (V - e X)
        f32x4 Y[4][CT];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KBK; ++kb) x = mma(x, frag_rows(Ks, L::LDK, 16 * tt, kb, lane), sh[kb][ct]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * tt + 4 * lg + i;
                    const float vv = ld_in(Vs + rr * L::LDV + wave * WC + 16 * ct + lr);
                    Y[tt][ct][i] = gB[rr] * (vv - gE[rr] * x[i]);
                }
            }
        // U = Y + T_off Y
        Frag yf[KBT][CT];
#pragma unroll
        for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                if constexpr (P::kBF16) yf[kb][ct] = bfrag_hi(Y[2 * kb][ct], Y[2 * kb + 1][ct]);
                else yf[kb][ct] = Y[kb][ct];
            }
        f32x4 U[4][CT];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int kmax = P::kBF16 ? tt / 2 : tt;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                U[tt][ct] = Y[tt][ct];
#pragma unroll
                for (int kb = 0; kb < KBT; ++kb)
                    if (kb <= kmax) U[tt][ct] = mma(U[tt][ct], frag_rows(Ts, L::LDT, 16 * tt, kb, lane), yf[kb][ct]);
            }
        }
        // U fragments for the output product
        if constexpr (WITH_O) {
            Frag uh[KBT][CT], ul[KBT][CT];
#pragma unroll
            for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    if constexpr (P::kBF16) bfrag_split(U[2 * kb][ct], U[2 * kb + 1][ct], uh[kb][ct], ul[kb][ct]);
                    else uh[kb][ct] = U[kb][ct];
                }
            // O = e (Q S) + Pd U + P_off U
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int kmax = P::kBF16 ? tt / 2 : tt;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < KBK; ++kb) {
                        const Frag qf = frag_rows(Qs, L::LDK, 16 * tt, kb, lane);
                        o = mma(o, qf, sh[kb][ct]);
                        if constexpr (P::kBF16) o = mma(o, qf, sl[kb][ct]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = 16 * tt + 4 * lg + i;
                        o[i] = gE[rr] * o[i] + gPd[rr] * U[tt][ct][i];
                    }
#pragma unroll
                    for (int kb = 0; kb < KBT; ++kb)
                        if (kb <= kmax) {
                            const Frag ph = frag_rows(Ph, L::LDT, 16 * tt, kb, lane);
                            o = mma(o, ph, uh[kb][ct]);
                            if constexpr (P::kBF16) {
                                o = mma(o, ph, ul[kb][ct]);
                                o = mma(o, frag_rows(Pl, L::LDT, 16 * tt, kb, lane), uh[kb][ct]);
                            }
                        }
                    // stage (scaled) for a row-contiguous store
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = 16 * tt + 4 * lg + i;
                        const int cc = wave * WC + 16 * ct + lr;
                        if (a.o_f32) Osf[rr * (W + 4) + cc] = a.scale * o[i];
                        else st_op(Os + rr * L::LDV + cc, a.scale * o[i]);
                    }
                }
            }
        }
        // S <- e_last S + K^T diag(G_last) U
        Frag dh[KBT][CT], dl[KBT][CT];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) U[tt][ct][i] *= gL[16 * tt + 4 * lg + i];
#pragma unroll
        for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                if constexpr (P::kBF16) bfrag_split(U[2 * kb][ct], U[2 * kb + 1][ct], dh[kb][ct], dl[kb][ct]);
                else dh[kb][ct] = U[kb][ct];
            }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                f32x4 s = S[rt][ct] * gam_c;
#pragma unroll
                for (int kb = 0; kb < KBT; ++kb) {
                    if constexpr (P::kBF16) {
                        const Frag kf = frag_rows(Kt, L::LDT, 16 * rt, kb, lane);
                        s = mma(s, kf, dh[kb][ct]);
                        s = mma(s, kf, dl[kb][ct]);
                    } else {
                        s = mma(s, frag_cols(reinterpret_cast<const float *>(Ks), L::LDK, 16 * rt, kb, lane),
                                dh[kb][ct]);
                    }
                }
                S[rt][ct] = s;
            }

        if constexpr (WITH_O) {
            if (a.o_out) {
                __syncthreads();
                // row-contiguous store of the staged outputs (rows < len)
                const int64_t obase = replay ? orow0 + c0 : t0;
                if (a.o_f32) {
                    constexpr int NV4 = W / 4;
                    float *og = reinterpret_cast<float *>(a.o_out);
                    for (int e = tid; e < CH * NV4; e += NTHR) {
                        const int rr = e / NV4, vc = e % NV4;
                        if (rr < len)
                            *reinterpret_cast<f32x4 *>(og + ((obase + rr) * a.h_v + h) * DV + cb * W + 4 * vc) =
                                *reinterpret_cast<const f32x4 *>(Osf + rr * (W + 4) + 4 * vc);
                    }
                } else {
                    E *og = reinterpret_cast<E *>(a.o_out);
                    for (int e = tid; e < CH * NVV; e += NTHR) {
                        const int rr = e / NVV, vc = e % NVV;
                        if (rr < len)
                            *reinterpret_cast<u32x4 *>(og + ((obase + rr) * a.h_v + h) * DV + cb * W + VEC * vc) =
                                *reinterpret_cast<const u32x4 *>(Os + rr * L::LDV + VEC * vc);
                    }
                }
            }
        }
    }

    // ---- state write-back
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.S_out[sbase + (int64_t)(16 * rt + 4 * lg + i) * DV + col0 + 16 * ct + lr] = S[rt][ct][i];
}

template <int DK, int DV, int W, class P, bool WITH_O>
hipError_t launch_t(const ChunkArgs &a, hipStream_t stream)
{
    const int64_t nblk = (int64_t)a.n_seqs * a.h_v * (DV / W);
    if (nblk <= 0) return hipSuccess;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gdn_chunk_kernel<DK, DV, W, P, WITH_O>), dim3((unsigned)nblk), dim3(NTHR), 0,
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
