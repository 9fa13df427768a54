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
    const float *S0;            // [n_seqs, h_v, d_k, d_v] initial state (prefill), nullable
    float *S_out;               // [n_seqs, h_v, d_k, d_v]
    void *o_out;                // [T_out, h_v, d_v], nullable
    int32_t *cu_out;            // [n_seqs + 1] output row offsets, nullable
    int32_t *status;            // device status word (workspace)
    int64_t total_tokens;
    int64_t total_out;          // rows of o_out (bounds every o store)
    int32_t n_seqs, h_qk, h_v;
    int32_t o_f32;              // o stored as fp32 (1) or in the input dtype (0)
    float scale;
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

constexpr int32_t kStatusOk = 0;
constexpr int32_t kStatusBadInput = 8;   // == GDN_ERR_DEVICE_INPUT

}  // namespace gdn
