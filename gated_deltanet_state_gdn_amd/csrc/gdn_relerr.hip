// Error report: relative Frobenius distance between two sets of recurrent states,
// ||S_a - S_b||_F / ||S_b||_F per state (||S_a||_F when ||S_b||_F = 0), with fp64
// accumulation, plus a count of non-finite entries of S_a.  It compares a rebuilt
// (replayed) state with the full-prefill state: Tail-Replay approximates the state
// at the prefix boundary by replaying a short recent suffix (arXiv 2608.30310,
// abstract), and this is the size of that approximation.
#include "gdn_common.h"

namespace gdn {
namespace {

constexpr int RT = 256;

__global__ void __launch_bounds__(RT) relerr_kernel(const float *A, const float *B, int32_t elems,
                                                    float *out, int32_t *nonfinite)
{
    __shared__ double sn[RT / 64], sd[RT / 64];
    __shared__ int sf[RT / 64];
    const int64_t s = blockIdx.x;
    const float *a = A + s * elems, *b = B + s * elems;
    double num = 0.0, den = 0.0;
    int nf = 0;
    for (int i = threadIdx.x * 4; i < elems; i += RT * 4) {
        // elems is a multiple of 4 (d_k, d_v in {64, 128}); 16-byte loads
        const float4 x = *reinterpret_cast<const float4 *>(a + i);
        const float4 y = *reinterpret_cast<const float4 *>(b + i);
        const float xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (!__builtin_isfinite(xs[j])) ++nf;
            const double d = (double)xs[j] - (double)ys[j];
            num += d * d;
            den += (double)ys[j] * (double)ys[j];
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        num += __shfl_xor(num, off);
        den += __shfl_xor(den, off);
        nf += __shfl_xor(nf, off);
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { sn[w] = num; sd[w] = den; sf[w] = nf; }
    __syncthreads();
    if (threadIdx.x == 0) {
        double tn = 0.0, td = 0.0;
        int tf = 0;
        for (int i = 0; i < RT / 64; ++i) { tn += sn[i]; td += sd[i]; tf += sf[i]; }
        out[s] = (float)(td > 0.0 ? sqrt(tn / td) : sqrt(tn));
        if (nonfinite) nonfinite[s] = tf;
    }
}

}  // namespace

hipError_t launch_relerr(const float *A, const float *B, int64_t n_states, int32_t elems,
                         float *relerr, int32_t *nonfinite, hipStream_t stream)
{
    if (n_states <= 0) return hipSuccess;
    if (n_states > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(relerr_kernel, dim3((unsigned)n_states), dim3(RT), 0, stream, A, B, elems,
                       relerr, nonfinite);
    return hipGetLastError();
}

}  // namespace gdn
