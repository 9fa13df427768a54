// Segment-parallel replay for gfx950: the pieces around the chunk kernel.
//
// The state recurrence of the gated delta rule (Gated DeltaNet) is affine in the state:
// over any stretch of tokens, S_end = M S_start + S_local, where S_local is the state the
// stretch builds from a zero start and M (d_k x d_k) is the product of the per-token maps
// alpha_t (I - beta_t k_t k_t^T) -- the same recurrence run from S_start = I with v = 0.
// A long replay window (Tail-Replay's last r tokens of a matched prefix) is cut into P
// chunk-aligned segments; one launch of the chunk kernel forms every segment's S_local and
// M at once (P times the parallelism of one window), the combine below chains them,
// S_start(p + 1) = M_p S_start(p) + S_local(p), S_start(0) = 0, in fp32, and a second
// chunk-kernel launch re-runs every segment from its true start to produce the outputs.
#include "gdn_common.h"

namespace gdn {
namespace {

constexpr int CHK = 64;   // chunk length of the chunk kernel (segments are chunk-aligned)

// Workgroup barrier that orders LDS only: global loads and stores stay in flight across
// it (a full __syncthreads also waits for every outstanding global access).
__device__ __forceinline__ void sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One block.  Virtual sequence v = n P + p is segment p of sequence n's window
// [end - r, end), cut at multiples of q = ceil(chunks / P) chunks; it is given to the chunk
// kernel as the packed range [vcu[v], vcu[v + 1]) with replay length vr[v] (its tokens are
// the last vr[v] of that range; segment 0's range starts at the sequence's own start, so
// the ranges tile the packed tokens).  Also the output row offsets of the real sequences
// (cu_out, nullable).  An invalid cu_seqlens / r entry sets the input bit of the status
// word and gives that sequence empty segments.
__global__ void __launch_bounds__(1024) seg_setup_kernel(const int32_t *cu, const int32_t *r, int32_t n_seqs,
                                                         int32_t P, int64_t total_tokens, int32_t *vcu,
                                                         int32_t *vr, int32_t *cu_out, int32_t *status)
{
    __shared__ int64_t part[16];
    const int t = threadIdx.x;
    const int64_t per = ((int64_t)n_seqs + 1023) / 1024;
    const int64_t m0 = (int64_t)t * per, m1 = (m0 + per < n_seqs) ? m0 + per : n_seqs;
    int bad = 0;
    int64_t sum = 0;
    int32_t keep[8];   // valid replay lengths of this thread's first 8 sequences
    for (int64_t m = m0; m < m1; ++m) {
        const int64_t b0 = cu[m], b1 = cu[m + 1];
        int64_t rr = r[m];
        const bool ok = b0 >= 0 && b1 >= b0 && b1 <= total_tokens && rr >= 0 && rr <= b1 - b0;
        if (!ok) {
            bad = 1;
            rr = 0;
        }
        if (m - m0 < 8) keep[m - m0] = (int32_t)rr;
        const int64_t wbeg = b1 - rr;
        const int64_t chunks = (rr + CHK - 1) / CHK;
        const int64_t q = (chunks + P - 1) / P;
        for (int p = 0; p < P; ++p) {
            int64_t s = wbeg + (int64_t)CHK * q * p, e = s + (int64_t)CHK * q;
            s = s < b1 ? s : b1;
            e = e < b1 ? e : b1;
            const int64_t v = m * P + p;
            vcu[v] = (int32_t)(p == 0 ? b0 : s);
            vr[v] = (int32_t)(e - s);
        }
        sum += rr;
    }
    if (t == 0) vcu[(int64_t)n_seqs * P] = n_seqs > 0 ? cu[n_seqs] : 0;
    // exclusive prefix of the thread ranges' sums: within each wave by shuffles, then over
    // the 16 wave totals
    const int lane = t & 63, wv = t >> 6;
    int64_t inc = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    if (lane == 63) part[wv] = inc;
    __syncthreads();
    if (t == 0) {
        int64_t acc = 0;
        for (int i = 0; i < 16; ++i) {
            const int64_t x = part[i];
            part[i] = acc;
            acc += x;
        }
    }
    __syncthreads();
    const int64_t excl = part[wv] + inc - sum;
    if (cu_out) {
        int64_t acc = excl;
        for (int64_t m = m0; m < m1; ++m) {
            cu_out[m] = (int32_t)acc;
            if (m - m0 < 8) {
                acc += keep[m - m0];
            } else {
                const int64_t b0 = cu[m], b1 = cu[m + 1];
                const int64_t rr = r[m];
                if (b0 >= 0 && b1 >= b0 && b1 <= total_tokens && rr >= 0 && rr <= b1 - b0) acc += rr;
            }
        }
        if (m1 == n_seqs && m0 < m1) cu_out[n_seqs] = (int32_t)acc;
        if (n_seqs == 0 && t == 0) cu_out[0] = 0;
    }
    if (bad) atomicOr(status, kStatusBitInput);
}

// Chain the segments of one (sequence, v-head) over a 16-column slice of S on the matrix
// cores, fp32 sums:
//     S = L_0;  Sstart[v_0] = 0;  for p = 1 .. P-1:  Sstart[v_p] = S;  S = M_p S + L_p;
//     S_out = S,
// v_p = n P + p.  L and M are the two halves of the map launch's states, each
// [n_seqs P, h_v, DK, DK]: L_p = S_local of segment p (row-major), M_p its transition map
// (16 x 16 tiles, tile (i, j) at 256 (i DK/16 + j), row-major inside).
//   SPLIT = false: 16x16x4 fp32 products (exact products), for fp32 inputs.
//   SPLIT = true (bf16 inputs, whose state is bounded by the fp16 range contract): every
//     operand x is split into fp16 hi = fp16(x) and lo = fp16(x - hi), and M S is formed
//     as hi*hi + hi*lo + lo*hi on 16x16x32 fp16 products: three matrix instructions per
//     32-wide k-block instead of eight 16x16x4 fp32 ones.  The dropped lo*lo and the roundings leave ~2e-7 of the step's result
//     M S + L, as an fp32 product would, also for decayed maps whose small entries have
//     fp16-subnormal lo halves (an absolute error of 2^-25 per entry, small against L).
//     S is split once, when it is written to LDS.
// Block: DK / 16 waves, one 16-row tile of the slice each; the M and L fragments of the
// next three steps are in flight while the current step's products run.  S lives in LDS
// transposed ([column][row], rows padded so that the 16 lanes reading one k-range of
// the 16 columns hit distinct banks), double-buffered across the steps.
template <int DK, bool SPLIT>
__global__ void __launch_bounds__(64 * (DK / 16)) seg_combine_kernel(const float *L, const float *M, float *Sstart,
                                                                     float *S_out, int32_t n_seqs, int32_t h_v,
                                                                     int32_t P)
{
    constexpr int LD = DK + 4;                 // padded row (one column of S) in LDS, fp32
    constexpr int LH = DK + 8;                 // the same for the fp16 halves
    constexpr int KB = DK / 16;                // 16-wide k-blocks (fp32 fragments)
    typedef __attribute__((ext_vector_type(4))) float f4;
    typedef __attribute__((ext_vector_type(8))) _Float16 h8;
    typedef __attribute__((ext_vector_type(2))) _Float16 h2;
    typedef __attribute__((ext_vector_type(2))) float f2;
    __shared__ __attribute__((aligned(16))) float st[2][16 * LD];
    __shared__ __attribute__((aligned(16))) _Float16 sth[SPLIT ? 2 : 1][SPLIT ? 16 * LH : 8];
    __shared__ __attribute__((aligned(16))) _Float16 stl[SPLIT ? 2 : 1][SPLIT ? 16 * LH : 8];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    // XCD-aware block order: the KB column slices of one (sequence, head) share an XCD
    // (blocks go round-robin over the 8 XCDs), so that M_p comes from HBM once per XCD
    // and the other slices find it in that XCD's L2
    const int64_t b = blockIdx.x;
    const int64_t slot = b >> 3;
    const int cs = (int)(slot % KB);           // column slice
    const int64_t nh = (slot / KB) * 8 + (b & 7);   // (sequence, head)
    if (nh >= (int64_t)n_seqs * h_v) return;   // padding of the last group of 8
    const int h = (int)(nh % h_v);
    const int64_t n = nh / h_v;
    const int c0 = 16 * cs, r0 = 16 * wave;
    const int64_t SS = (int64_t)DK * DK;       // floats per state
    auto state_at = [&](int p) { return ((n * P + p) * h_v + h) * SS; };
    // this lane's part of S_new = M_p S + L_p: rows r0 + 4 (l/16) + i, column c0 + l%16.
    // M_p fragments, row r0 + l%16, columns 16 kb + 4 (l/16) .. +3 of each 16-wide block:
    // each load reads one whole 1 KB tile.  The split products take the fragments of
    // blocks 2 j and 2 j + 1 as the eight k values of one 16x16x32 product, i.e. lane
    // group g contracts over columns 32 j + 4 g .. +3 and 32 j + 16 + 4 g .. +3 (the S
    // fragments are read from LDS in the same order).  Three register sets keep the operands of steps p + 1 ..
    // p + 3 in flight while step p runs; a set is refilled only once its step has consumed
    // it, so the loop carries each set in the same registers (no copies that would wait
    // for the loads just issued).
    struct Ops {
        f4 m[KB];
        f4 l;
    };
    auto load = [&](Ops &o, int p) {
        const int64_t base = state_at(p);
        // (M is stored as 16 x 16 tiles)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            o.m[kb] = *reinterpret_cast<const f4 *>(M + base + (int64_t)(wave * KB + kb) * 256 + 16 * lr + 4 * lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) o.l[i] = L[base + (int64_t)(r0 + 4 * lg + i) * DK + c0 + lr];
    };
    // the new S (this lane's four entries) into buffer q: fp32, and for SPLIT its halves
    auto put_s = [&](int q, f4 x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st[q][lr * LD + r0 + 4 * lg + i] = x[i];
        if constexpr (SPLIT) {
            h2 h01 = __builtin_convertvector(f2{x[0], x[1]}, h2), h23 = __builtin_convertvector(f2{x[2], x[3]}, h2);
            const f2 b01 = __builtin_convertvector(h01, f2), b23 = __builtin_convertvector(h23, f2);
            const h2 l01 = __builtin_convertvector(f2{x[0] - b01[0], x[1] - b01[1]}, h2);
            const h2 l23 = __builtin_convertvector(f2{x[2] - b23[0], x[3] - b23[1]}, h2);
            typedef __attribute__((ext_vector_type(4))) _Float16 h4;
            *reinterpret_cast<h4 *>(&sth[q][lr * LH + r0 + 4 * lg]) = h4{h01[0], h01[1], h23[0], h23[1]};
            *reinterpret_cast<h4 *>(&stl[q][lr * LH + r0 + 4 * lg]) = h4{l01[0], l01[1], l23[0], l23[1]};
        }
    };
    // (the 16 columns of one row: 4 consecutive per lane group, from the transposed copy)
    auto put_rows = [&](float *dst, const float *src) {
        f4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = src[(4 * lg + j) * LD + r0 + lr];
        *reinterpret_cast<f4 *>(dst + (int64_t)(r0 + lr) * DK + c0 + 4 * lg) = x;
    };
    int cur = 0;
    // one step: Sstart[v_p] = S, S = M_p S + L_p, then the operands of step p + 3 into o
    auto step = [&](Ops &o, int p) {
        put_rows(Sstart + state_at(p), st[cur]);
        f4 acc = o.l;
        if constexpr (SPLIT) {
            h8 ah[KB / 2], al[KB / 2];
#pragma unroll
            for (int j = 0; j < KB / 2; ++j) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = o.m[2 * j + (e >> 2)][e & 3];
                    ah[j][e] = (_Float16)x;
                    al[j][e] = (_Float16)(x - (float)ah[j][e]);
                }
            }
#pragma unroll
            for (int j = 0; j < KB / 2; ++j) {
                typedef __attribute__((ext_vector_type(4))) _Float16 h4;
                const int k0 = lr * LH + 32 * j + 4 * lg;
                const h4 bh0 = *reinterpret_cast<const h4 *>(&sth[cur][k0]);
                const h4 bh1 = *reinterpret_cast<const h4 *>(&sth[cur][k0 + 16]);
                const h4 bl0 = *reinterpret_cast<const h4 *>(&stl[cur][k0]);
                const h4 bl1 = *reinterpret_cast<const h4 *>(&stl[cur][k0 + 16]);
                const h8 bh = __builtin_shufflevector(bh0, bh1, 0, 1, 2, 3, 4, 5, 6, 7);
                const h8 bl = __builtin_shufflevector(bl0, bl1, 0, 1, 2, 3, 4, 5, 6, 7);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[j], bh, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[j], bl, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[j], bh, acc, 0, 0, 0);
            }
        } else {
            // every S fragment first, then two independent product chains (even and odd
            // k-blocks), summed at the end
            f4 bf[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) bf[kb] = *reinterpret_cast<const f4 *>(&st[cur][lr * LD + 16 * kb + 4 * lg]);
            f4 acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; kb += 2) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(o.m[kb][j], bf[kb][j], acc, 0, 0, 0);
                    acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(o.m[kb + 1][j], bf[kb + 1][j], acc2, 0, 0, 0);
                }
            }
            acc += acc2;
        }
        put_s(cur ^ 1, acc);
        // (after the products: the registers of o, acc's start included, are free again;
        // unconditional, no branch around the loads)
        load(o, p + 3 < P ? p + 3 : P - 1);
        sync_lds();
        cur ^= 1;
    };

    Ops A, B, C;
    // segment 0 starts from zero: S = L_0, no product
    {
        f4 z = {0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f4 *>(Sstart + state_at(0) + (int64_t)(r0 + lr) * DK + c0 + 4 * lg) = z;
        const int64_t base = state_at(0);
        f4 l0;
#pragma unroll
        for (int i = 0; i < 4; ++i) l0[i] = L[base + (int64_t)(r0 + 4 * lg + i) * DK + c0 + lr];
        put_s(0, l0);
    }
    if (P > 1) {
        load(A, 1);
        load(B, P > 2 ? 2 : P - 1);
        load(C, P > 3 ? 3 : P - 1);
    }
    sync_lds();
    // whole triples in the loop (every path round it runs all three steps, so the wait
    // for a set's loads never has to assume the other two sets were skipped), then the rest
    int p = 1;
    for (; p + 2 < P; p += 3) {
        step(A, p);
        step(B, p + 1);
        step(C, p + 2);
    }
    if (p < P) step(A, p);
    if (p + 1 < P) step(B, p + 1);
    put_rows(S_out + (n * h_v + h) * SS, st[cur]);
}

}  // namespace

hipError_t launch_seg_setup(const int32_t *cu, const int32_t *r, int32_t n_seqs, int32_t P,
                            int64_t total_tokens, int32_t *vcu, int32_t *vr, int32_t *cu_out,
                            int32_t *status, hipStream_t stream)
{
    hipLaunchKernelGGL(seg_setup_kernel, dim3(1), dim3(1024), 0, stream, cu, r, n_seqs, P, total_tokens, vcu,
                       vr, cu_out, status);
    return hipGetLastError();
}

hipError_t launch_seg_combine(const float *L, const float *M, float *Sstart, float *S_out, int32_t n_seqs,
                              int32_t h_v, int32_t d, int32_t P, bool split, hipStream_t stream)
{
    // (sequence, head) pairs rounded up to a multiple of 8 (the XCD grouping)
    const int64_t blocks = (((int64_t)n_seqs * h_v + 7) / 8) * 8 * (d / 16);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
#define GDN_COMBINE(D, SPL)                                                                             \
    hipLaunchKernelGGL((seg_combine_kernel<D, SPL>), dim3((unsigned)blocks), dim3(4 * D), 0, stream, L, M, \
                       Sstart, S_out, n_seqs, h_v, P)
    if (d == 128) {
        if (split) GDN_COMBINE(128, true);
        else GDN_COMBINE(128, false);
    } else if (d == 64) {
        if (split) GDN_COMBINE(64, true);
        else GDN_COMBINE(64, false);
    } else {
        return hipErrorNotSupported;
    }
#undef GDN_COMBINE
    return hipGetLastError();
}

}  // namespace gdn
