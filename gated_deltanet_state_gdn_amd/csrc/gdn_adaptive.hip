// Adaptive replay length: per sequence, the shortest tail whose gates have attenuated
// every v-head's older state below a tolerance.
//
// Replaying the last r tokens from a zero state differs from the full recurrence by
// the propagated older state, M S_before with M the product of the r per-token maps
// alpha_t (I - beta_t k_t k_t^T).  For unit keys and beta in [0, 1] each map has
// spectral norm at most alpha_t, so the error is at most (prod alpha_t) ||S_before||
// (Tail-Replay, arXiv 2608.30310: the gated updates progressively attenuate the
// influence of distant tokens, which is why a short recent window suffices).  The
// pages replay a fixed fraction of the prefix; this picks, per sequence, the
// smallest r for which prod alpha_t = exp(sum g_t) over the window is at most eps
// for every v-head.
//
// The decision is exact integer arithmetic: each g is rounded once to a multiple of
// 2^-32 nats, windows are summed in int64 (saturating at -2^53, far below any
// threshold, which leaves every comparison unchanged since all terms are <= 0), and
// compared with floor(ln(eps) * 2^32) computed on the host.  Any summation order
// therefore gives the same r.
//
// Pass 1: one wavefront per (sequence, v-head) walks the sequence backwards, 512
// tokens per step (8 per lane, in flight together), with a wavefront prefix sum,
// and stops at the first crossing.  Pass 2: one workgroup takes the maximum over
// heads, clamps it, validates cu_seqlens and sets the status word's bad-input bit.
#include <atomic>
#include <mutex>

#include "gdn_common.h"

namespace gdn {

// Device memory of the allocation-free variant (gdn_adaptive_replay_len_static): word 0
// is its status word, words [kStaticPad, kStaticPad + kStaticHeads) its per-head
// lengths.  Every GPU the library runs on holds its own copy until the process ends.
// Host code never uses this name as an address: static_scratch() returns the device
// address, looked up once per device.
constexpr int kStaticPad = 64;                      // status word, padded to 256 bytes
static __device__ __align__(256) int32_t scratch[kStaticPad + kStaticHeads];

namespace {

constexpr int U = 8;                              // tokens per lane per step
constexpr int64_t kSat = -(int64_t(1) << 53);     // saturation floor of partial sums
constexpr int64_t kReset = -(int64_t(1) << 52);   // a gate at or below -2^20 nats

__device__ __forceinline__ int64_t sat_add(int64_t a, int64_t b) {
    const int64_t s = a + b;                      // both >= kSat: no overflow
    return s < kSat ? kSat : s;
}

// g in nats -> multiple of 2^-32 nats (exact for |g| < 2^20)
__device__ __forceinline__ int64_t quant(float g) {
    const double x = (double)g;
    if (!(x < 0.0)) return 0;                     // g >= 0 or NaN: no attenuation
    if (x <= -1048576.0) return kReset;           // includes -inf (alpha = 0)
    return (int64_t)rint(x * 4294967296.0);
}

__global__ void __launch_bounds__(256) adaptive_head_kernel(const float *g, const int32_t *cu,
                                                            int32_t n_seqs, int32_t h_v,
                                                            int64_t total, int64_t thr,
                                                            int32_t r_max, int32_t *r_head)
{
    const int lane = threadIdx.x & 63;
    const int64_t job = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (job >= (int64_t)n_seqs * h_v) return;
    const int n = (int)(job / h_v), h = (int)(job % h_v);
    const int64_t b = cu[n], e = cu[n + 1];
    if (b < 0 || e < b || e > total) {
        if (lane == 0) r_head[job] = 0;
        return;
    }
    const int64_t lim = e - b < (int64_t)r_max ? e - b : (int64_t)r_max;
    int64_t r_h = lim;
    if (thr >= 0) {
        r_h = 0;                                  // the empty window already qualifies
    } else {
        int64_t run = 0;
        for (int64_t base = 0; base < lim; base += 64 * U) {
            int64_t p[U];
            const int64_t d0 = base + (int64_t)lane * U;   // depth from the end
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int64_t d = d0 + i;
                p[i] = d < lim ? quant(g[(e - 1 - d) * h_v + h]) : 0;
            }
#pragma unroll
            for (int i = 1; i < U; ++i) p[i] = sat_add(p[i], p[i - 1]);
            // inclusive wavefront scan of the lane totals
            int64_t inc = p[U - 1];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int64_t y = __shfl_up(inc, off);
                if (lane >= off) inc = sat_add(inc, y);
            }
            // exclusive prefix of this lane = inclusive scan of the previous lane
            int64_t ex = __shfl_up(inc, 1);
            if (lane == 0) ex = 0;
            const int64_t start = sat_add(run, ex);
            int first = U;
#pragma unroll
            for (int i = U - 1; i >= 0; --i)
                if (d0 + i < lim && sat_add(start, p[i]) <= thr) first = i;
            const unsigned long long hit = __ballot(first < U);
            if (hit) {
                const int l = __ffsll((long long)hit) - 1;
                const int fi = __shfl(first, l);
                r_h = base + (int64_t)l * U + fi + 1;
                break;
            }
            run = sat_add(run, __shfl(inc, 63));
        }
    }
    if (lane == 0) r_head[job] = (int32_t)r_h;
}

__global__ void __launch_bounds__(256) adaptive_reduce_kernel(const int32_t *cu, int32_t n_seqs,
                                                              int32_t h_v, int64_t total,
                                                              int32_t r_min, int32_t r_max,
                                                              const int32_t *r_head,
                                                              int32_t *r_out, int32_t *status)
{
    int bad = 0;
    for (int n = threadIdx.x; n < n_seqs; n += blockDim.x) {
        const int64_t b = cu[n], e = cu[n + 1];
        if (b < 0 || e < b || e > total) {
            bad = 1;
            r_out[n] = 0;
            continue;
        }
        int64_t m = 0;
        for (int h = 0; h < h_v; ++h) {
            const int64_t x = r_head[(int64_t)n * h_v + h];
            m = x > m ? x : m;
        }
        const int64_t L = e - b;
        const int64_t lo = (int64_t)r_min < L ? (int64_t)r_min : L;
        const int64_t hi = (int64_t)r_max < L ? (int64_t)r_max : L;
        m = m < lo ? lo : m;
        m = m > hi ? hi : m;
        r_out[n] = (int32_t)m;
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0 && bad) atomicOr(status, kStatusBitInput);
}

}  // namespace

// Device address of `scratch` on the current device, looked up on the first call with
// that device current and kept per device; nullptr if the lookup fails.
static int32_t *static_scratch()
{
    static std::mutex mu;
    static int32_t *addr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev] = static_cast<int32_t *>(p);
    }
    return addr[dev];
}

hipError_t launch_adaptive_static(const float *g, const int32_t *cu, int32_t n_seqs, int32_t h_v,
                                  int64_t total_tokens, int64_t thr, int32_t r_min, int32_t r_max,
                                  int32_t *r_out, hipStream_t stream)
{
    if ((int64_t)n_seqs * h_v > kStaticHeads) return hipErrorInvalidValue;
    int32_t *base = static_scratch();
    if (!base) return hipErrorInvalidSymbol;
    // the per-head lengths are all written by the first kernel before the second reads
    // them, so nothing needs clearing; the status word only collects bits nobody reads
    // (a bad cu_seqlens shows as r_out[n] = 0)
    return launch_adaptive(g, cu, n_seqs, h_v, total_tokens, thr, r_min, r_max, base + kStaticPad,
                           r_out, base, stream);
}

hipError_t launch_adaptive(const float *g, const int32_t *cu, int32_t n_seqs, int32_t h_v,
                           int64_t total_tokens, int64_t thr, int32_t r_min, int32_t r_max,
                           int32_t *r_head, int32_t *r_out, int32_t *status, hipStream_t stream)
{
    const int64_t jobs = (int64_t)n_seqs * h_v;
    if (jobs > 0) {
        const int64_t blocks = (jobs + 3) / 4;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(adaptive_head_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g,
                           cu, n_seqs, h_v, total_tokens, thr, r_max, r_head);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(adaptive_reduce_kernel, dim3(1), dim3(256), 0, stream, cu, n_seqs, h_v,
                       total_tokens, r_min, r_max, r_head, r_out, status);
    return hipGetLastError();
}

}  // namespace gdn
