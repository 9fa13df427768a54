// Internal declarations shared by the C-ABI host code and the gfx950 kernels.
// Not part of the public interface (that is include/gdn.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Arguments of the chunked gated-delta-rule kernel (one launch covers every
// (sequence, v-head) chain of a call).
struct ChunkArgs {
    const void *q, *k, *v;      // [T, h_qk, d_k], [T, h_qk, d_k], [T, h_v, d_v]
    const float *g, *beta;      // [T, h_v]
    const int32_t *cu;          // [n_seqs + 1]
    const int32_t *r;           // [n_seqs], replay lengths; nullptr = full prefill
    const float *S0;            // [n_seqs, h_v, d_k, d_v] initial state, nullable (zero)
    float *S_out;               // [n_seqs, h_v, d_k, d_v]
    void *o_out;                // [T_out, h_v, d_v], nullable
    int32_t *cu_out;            // [n_seqs + 1] output row offsets, nullable
    int32_t *status;            // device status word (workspace)
    int64_t total_tokens;
    int64_t total_out;          // rows of o_out (bounds every o store)
    int32_t n_seqs, h_qk, h_v;
    int32_t o_f32;              // o stored as fp32 (1) or in the input dtype (0)
    float scale;
    // 1: every sequence also has h_v transition-map units (V read as zero, S started at
    // the identity; square states, no outputs), whose final states follow the n_seqs h_v
    // usual ones in S_out: [2, n_seqs, h_v, d_k, d_k], the maps as 16 x 16 tiles (tile
    // (i, j) at 256 (i d_k/16 + j) floats, row-major inside)
    int32_t mpart = 0;
    // grid plan (set by the launcher): blocks [0, n_full) take whole work units, the
    // rest take 1/2^split of a unit's columns each
    int64_t n_full;
    int32_t split;
};

// Launch the chunk kernel (state waves and prep waves on double-buffered LDS) for the
// given dtype / head dims.  Returns hipSuccess or the launch error;
// hipErrorNotSupported for an unsupported combination.
hipError_t launch_chunk_ws(const ChunkArgs &a, int bf16, int d_k, int d_v, bool with_o,
                           hipStream_t stream);

hipError_t launch_relerr(const float *A, const float *B, int64_t n_states, int32_t elems,
                         float *relerr, int32_t *nonfinite, hipStream_t stream);

// Adaptive replay length: r_head [n_seqs * h_v] is scratch (per-head lengths), r_out
// [n_seqs] the clamped per-sequence maximum; thr = floor(ln(eps) * 2^32).
hipError_t launch_adaptive(const float *g, const int32_t *cu, int32_t n_seqs, int32_t h_v,
                           int64_t total_tokens, int64_t thr, int32_t r_min, int32_t r_max,
                           int32_t *r_head, int32_t *r_out, int32_t *status, hipStream_t stream);

// The same with the per-head lengths and the status word in the library's static device
// scratch (no workspace, no allocation).  n_seqs * h_v must be <= kStaticHeads
// (hipErrorInvalidValue otherwise); hipErrorInvalidSymbol if the scratch's device address
// cannot be looked up.
constexpr int64_t kStaticHeads = 65536;
hipError_t launch_adaptive_static(const float *g, const int32_t *cu, int32_t n_seqs, int32_t h_v,
                                  int64_t total_tokens, int64_t thr, int32_t r_min, int32_t r_max,
                                  int32_t *r_out, hipStream_t stream);

// Segment-parallel replay (gdn_segment.hip).  Setup: virtual sequences v = n P + p (segment
// p of sequence n's window) as packed ranges vcu [n_seqs P + 1] and replay lengths vr
// [n_seqs P], plus the real output row offsets cu_out [n_seqs + 1] (nullable).
hipError_t launch_seg_setup(const int32_t *cu, const int32_t *r, int32_t n_seqs, int32_t P,
                            int64_t total_tokens, int32_t *vcu, int32_t *vr, int32_t *cu_out,
                            int32_t *status, hipStream_t stream);
// Combine: L, M = the map launch's states [n_seqs P, h_v, d, d] each; Sstart [n_seqs P, h_v,
// d, d] receives every segment's true start state, S_out [n_seqs, h_v, d, d] the final one.
// split: products on fp16 hi/lo halves (bf16 inputs) instead of fp32 ones.
hipError_t launch_seg_combine(const float *L, const float *M, float *Sstart, float *S_out, int32_t n_seqs,
                              int32_t h_v, int32_t d, int32_t P, bool split, hipStream_t stream);

// Bits of the device status word (workspace word 0).  Kernels only ever OR bits in
// (atomically); gdn_device_status reads the word and clears it.
constexpr int32_t kStatusBitInput = 1;   // cu_seqlens / r invalid  -> GDN_ERR_DEVICE_INPUT
constexpr int32_t kStatusBitWait = 2;    // a bounded in-workgroup wait expired -> GDN_ERR_DEVICE_WAIT

}  // namespace gdn
